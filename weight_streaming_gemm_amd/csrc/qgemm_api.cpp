// qgemm_api.cpp — host side of the C ABI: argument validation, the
// R-dependent launch plan, workspace ownership and the graph-captured pass.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <map>
#include <new>
#include <vector>

#include "../../include/qgemm.h"
#include "layout.h"
#include "qgemm_internal.h"

using namespace qg;

struct qgemm_handle {
  uint32_t magic;
  const uint8_t* packed;
  int64_t N, K, KB, NS;
  int max_R;
  int cus;
  // workspace (owned)
  void* xq;
  void* xs;
  float* part;
  size_t xq_bytes, xs_bytes, part_bytes;
};

static const uint32_t HANDLE_MAGIC = 0x51474D31u;  // "QGM1"
static const uint32_t SEQ_MAGIC = 0x51475331u;     // "QGS1"

namespace {

struct Plan {
  int path;
  int RT, NT, S;
  int64_t kbs;
  int64_t waves;
  int kernels;
  size_t ws_bytes;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_shape(int64_t N, int64_t K) {
  if (N < 1 || K < 256 || K % 256 != 0) return false;
  // packed bytes and N*K must fit comfortably in 64-bit arithmetic
  if (N > (int64_t(1) << 40) / 1 || K > (int64_t(1) << 30)) return false;
  if ((padded_n(N) / 16) * (K / 256) > (int64_t(1) << 40)) return false;
  return true;
}

bool valid_handle(const qgemm_handle* h) { return h && h->magic == HANDLE_MAGIC; }

// Matrix-core plan: row tiles of 16, NT sub-tiles per wave, and a K split that
// brings the number of waves near two per SIMD of the device (so every CU has
// work and the tail is short), with no split smaller than one block.
Plan plan_mfma(int64_t NS, int64_t KB, int64_t N, int R, int cus) {
  Plan p{};
  p.path = QGEMM_PATH_MFMA;
  p.RT = (R + 15) / 16;
  p.NT = (p.RT == 1) ? 2 : 1;
  int64_t NG = (NS + p.NT - 1) / p.NT;
  int64_t target = (int64_t)cus * 4 * 2;
  int64_t S = (target + NG / 2) / NG;
  if (S < 1) S = 1;
  if (S > KB) S = KB;
  p.kbs = (KB + S - 1) / S;
  p.S = (int)((KB + p.kbs - 1) / p.kbs);
  p.waves = NG * p.S;
  p.kernels = (p.S > 1) ? 3 : 2;
  p.ws_bytes = (size_t)p.RT * KB * 8 * 64 * 16 + (size_t)p.RT * KB * 64 * 8 +
               (p.S > 1 ? (size_t)p.S * R * N * 4 : 0);
  return p;
}

int make_plan(const qgemm_handle* h, int R, int path, Plan* out) {
  if (path == QGEMM_PATH_VALU) return QGEMM_EPATH;
  if (path != QGEMM_PATH_AUTO && path != QGEMM_PATH_MFMA) return QGEMM_EINVAL;
  *out = plan_mfma(h->NS, h->KB, h->N, R, h->cus);
  return QGEMM_OK;
}

int run_impl(qgemm_handle* h, const void* x, float* y, int R, int path, hipStream_t st) {
  Plan p;
  int rc = make_plan(h, R, path, &p);
  if (rc) return rc;
  hipError_t e = launch_xprep(reinterpret_cast<const uint16_t*>(x), h->xq, h->xs, R, h->K, p.RT, st);
  if (e != hipSuccess) return QGEMM_EHIP;
  MfmaArgs a{};
  a.packed = h->packed;
  a.xq = h->xq;
  a.xs = h->xs;
  a.out = (p.S > 1) ? h->part : y;
  a.N = h->N;
  a.KB = h->KB;
  a.NS = h->NS;
  a.R = R;
  a.S = p.S;
  a.RT = p.RT;
  a.NT = p.NT;
  a.kbs = p.kbs;
  a.hdr_off = quant_region_bytes(h->N, h->K);
  e = launch_mfma(a, st);
  if (e != hipSuccess) return QGEMM_EHIP;
  if (p.S > 1) {
    e = launch_reduce(h->part, y, (int64_t)R * h->N, p.S, st);
    if (e != hipSuccess) return QGEMM_EHIP;
  }
  return QGEMM_OK;
}

}  // namespace

extern "C" {

const char* qgemm_status_string(int status) {
  switch (status) {
    case QGEMM_OK: return "ok";
    case QGEMM_EINVAL: return "invalid argument (null pointer, bad handle or flag)";
    case QGEMM_ESHAPE: return "bad shape (K must be a positive multiple of 256, N >= 1)";
    case QGEMM_EALIGN: return "device pointer not 16-byte aligned";
    case QGEMM_ERANGE_R: return "row count out of range";
    case QGEMM_ENOMEM: return "out of device memory";
    case QGEMM_EHIP: return "HIP call or kernel launch failed";
    case QGEMM_EPATH: return "kernel path cannot serve this row count";
    default: return "unknown status";
  }
}

int qgemm_packed_size(int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return QGEMM_EINVAL;
  if (!valid_shape(N, K)) return QGEMM_ESHAPE;
  *bytes = (size_t)packed_bytes(N, K);
  return QGEMM_OK;
}

int qgemm_pack(const void* canon_dev, void* packed_dev, int64_t N, int64_t K, void* stream) {
  if (!canon_dev || !packed_dev) return QGEMM_EINVAL;
  if (!valid_shape(N, K)) return QGEMM_ESHAPE;
  if (!aligned16(canon_dev) || !aligned16(packed_dev)) return QGEMM_EALIGN;
  hipError_t e = launch_pack(reinterpret_cast<const uint8_t*>(canon_dev), reinterpret_cast<uint8_t*>(packed_dev),
                             N, K, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? QGEMM_OK : QGEMM_EHIP;
}

int qgemm_create(qgemm_t* out, const void* packed_dev, int64_t N, int64_t K, int max_R, uint32_t flags) {
  if (!out || !packed_dev || flags != 0) return QGEMM_EINVAL;
  *out = nullptr;
  if (!valid_shape(N, K)) return QGEMM_ESHAPE;
  if (!aligned16(packed_dev)) return QGEMM_EALIGN;
  if (max_R < 1 || max_R > QGEMM_MAX_R) return QGEMM_ERANGE_R;
  qgemm_handle* h = new (std::nothrow) qgemm_handle{};
  if (!h) return QGEMM_ENOMEM;
  h->magic = HANDLE_MAGIC;
  h->packed = reinterpret_cast<const uint8_t*>(packed_dev);
  h->N = N;
  h->K = K;
  h->KB = K / 256;
  h->NS = padded_n(N) / 16;
  h->max_R = max_R;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    delete h;
    return QGEMM_EHIP;
  }
  h->cus = cus;
  int rt_max = (max_R + 15) / 16;
  h->xq_bytes = (size_t)rt_max * h->KB * 8 * 64 * 16;
  h->xs_bytes = (size_t)rt_max * h->KB * 64 * 8;
  size_t part = 0;
  for (int R = 1; R <= max_R; ++R) {
    Plan p = plan_mfma(h->NS, h->KB, N, R, cus);
    if (p.S > 1) part = std::max(part, (size_t)p.S * R * N * 4);
  }
  h->part_bytes = part;
  if (hipMalloc(&h->xq, h->xq_bytes) != hipSuccess || hipMalloc(&h->xs, h->xs_bytes) != hipSuccess ||
      (part && hipMalloc(reinterpret_cast<void**>(&h->part), part) != hipSuccess)) {
    (void)hipGetLastError();
    if (h->xq) (void)hipFree(h->xq);
    if (h->xs) (void)hipFree(h->xs);
    if (h->part) (void)hipFree(h->part);
    delete h;
    return QGEMM_ENOMEM;
  }
  *out = h;
  return QGEMM_OK;
}

int qgemm_run_path(qgemm_t h, const void* x_bf16, float* y, int R, int path, void* stream) {
  if (!valid_handle(h)) return QGEMM_EINVAL;
  if (R < 0 || R > h->max_R) return QGEMM_ERANGE_R;
  if (path < QGEMM_PATH_AUTO || path > QGEMM_PATH_MFMA) return QGEMM_EINVAL;
  if (R == 0) return QGEMM_OK;
  if (!x_bf16 || !y) return QGEMM_EINVAL;
  if (!aligned16(x_bf16) || !aligned16(y)) return QGEMM_EALIGN;
  return run_impl(h, x_bf16, y, R, path, reinterpret_cast<hipStream_t>(stream));
}

int qgemm_run(qgemm_t h, const void* x_bf16, float* y, int R, void* stream) {
  return qgemm_run_path(h, x_bf16, y, R, QGEMM_PATH_AUTO, stream);
}

int qgemm_dequantize(qgemm_t h, float* w_out, void* stream) {
  if (!valid_handle(h) || !w_out) return QGEMM_EINVAL;
  if (!aligned16(w_out)) return QGEMM_EALIGN;
  hipError_t e = launch_dequant(h->packed, w_out, h->N, h->K, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? QGEMM_OK : QGEMM_EHIP;
}

int qgemm_argmax_rows(const float* y, int R, int64_t N, int32_t* idx, void* stream) {
  if (R < 0) return QGEMM_ERANGE_R;
  if (N < 1) return QGEMM_ESHAPE;
  if (R == 0) return QGEMM_OK;
  if (!y || !idx) return QGEMM_EINVAL;
  hipError_t e = launch_argmax(y, R, N, idx, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? QGEMM_OK : QGEMM_EHIP;
}

int qgemm_query(qgemm_t h, int R, int path, qgemm_info* info) {
  if (!valid_handle(h) || !info) return QGEMM_EINVAL;
  if (R < 1 || R > h->max_R) return QGEMM_ERANGE_R;
  Plan p;
  int rc = make_plan(h, R, path, &p);
  if (rc) return rc;
  info->path = p.path;
  info->split_k = p.S;
  info->row_tiles = p.RT;
  info->subtiles_per_wave = p.NT;
  info->waves = p.waves;
  info->kernels = p.kernels;
  info->workspace_bytes = p.ws_bytes;
  return QGEMM_OK;
}

int qgemm_destroy(qgemm_t h) {
  if (!h) return QGEMM_OK;
  if (!valid_handle(h)) return QGEMM_EINVAL;
  (void)hipDeviceSynchronize();
  if (h->xq) (void)hipFree(h->xq);
  if (h->xs) (void)hipFree(h->xs);
  if (h->part) (void)hipFree(h->part);
  h->magic = 0;
  delete h;
  return QGEMM_OK;
}

}  // extern "C"

// ---- full weight pass --------------------------------------------------------

struct GraphKey {
  int R;
  std::vector<uintptr_t> ptrs;
  bool operator<(const GraphKey& o) const {
    if (R != o.R) return R < o.R;
    return ptrs < o.ptrs;
  }
};

struct qgemm_seq {
  uint32_t magic;
  std::vector<qgemm_handle*> hs;
  hipStream_t cap;
  std::map<GraphKey, hipGraphExec_t> graphs;
};

extern "C" {

int qgemm_seq_create(qgemm_seq_t* out, const qgemm_t* handles, int count) {
  if (!out || !handles || count < 1) return QGEMM_EINVAL;
  *out = nullptr;
  for (int i = 0; i < count; ++i)
    if (!valid_handle(handles[i])) return QGEMM_EINVAL;
  qgemm_seq* s = new (std::nothrow) qgemm_seq{};
  if (!s) return QGEMM_ENOMEM;
  s->magic = SEQ_MAGIC;
  s->hs.assign(handles, handles + count);
  if (hipStreamCreateWithFlags(&s->cap, hipStreamNonBlocking) != hipSuccess) {
    delete s;
    return QGEMM_EHIP;
  }
  *out = s;
  return QGEMM_OK;
}

int qgemm_seq_run(qgemm_seq_t s, const void* const* xs, float* const* ys, int R, int32_t* argmax_idx,
                  void* stream) {
  if (!s || s->magic != SEQ_MAGIC || !xs || !ys) return QGEMM_EINVAL;
  if (R < 0) return QGEMM_ERANGE_R;
  for (size_t i = 0; i < s->hs.size(); ++i) {
    if (R > s->hs[i]->max_R) return QGEMM_ERANGE_R;
    if (R > 0 && (!xs[i] || !ys[i])) return QGEMM_EINVAL;
    if (R > 0 && (!aligned16(xs[i]) || !aligned16(ys[i]))) return QGEMM_EALIGN;
  }
  if (R == 0) return QGEMM_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  GraphKey key{R, {}};
  for (size_t i = 0; i < s->hs.size(); ++i) {
    key.ptrs.push_back(reinterpret_cast<uintptr_t>(xs[i]));
    key.ptrs.push_back(reinterpret_cast<uintptr_t>(ys[i]));
  }
  key.ptrs.push_back(reinterpret_cast<uintptr_t>(argmax_idx));
  auto it = s->graphs.find(key);
  if (it == s->graphs.end()) {
    if (hipStreamBeginCapture(s->cap, hipStreamCaptureModeThreadLocal) != hipSuccess) return QGEMM_EHIP;
    int rc = QGEMM_OK;
    for (size_t i = 0; i < s->hs.size() && rc == QGEMM_OK; ++i)
      rc = run_impl(s->hs[i], xs[i], ys[i], R, QGEMM_PATH_AUTO, s->cap);
    if (rc == QGEMM_OK && argmax_idx) {
      qgemm_handle* last = s->hs.back();
      if (launch_argmax(ys[s->hs.size() - 1], R, last->N, argmax_idx, s->cap) != hipSuccess) rc = QGEMM_EHIP;
    }
    hipGraph_t g = nullptr;
    hipError_t e = hipStreamEndCapture(s->cap, &g);
    if (rc != QGEMM_OK) {
      if (g) (void)hipGraphDestroy(g);
      return rc;
    }
    if (e != hipSuccess || !g) return QGEMM_EHIP;
    hipGraphExec_t ex = nullptr;
    e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if (e != hipSuccess) return QGEMM_EHIP;
    it = s->graphs.emplace(key, ex).first;
  }
  return hipGraphLaunch(it->second, st) == hipSuccess ? QGEMM_OK : QGEMM_EHIP;
}

int qgemm_seq_destroy(qgemm_seq_t s) {
  if (!s) return QGEMM_OK;
  if (s->magic != SEQ_MAGIC) return QGEMM_EINVAL;
  (void)hipDeviceSynchronize();
  for (auto& kv : s->graphs) (void)hipGraphExecDestroy(kv.second);
  (void)hipStreamDestroy(s->cap);
  s->magic = 0;
  delete s;
  return QGEMM_OK;
}

}  // extern "C"
