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
  int occ[5][5];  // resident workgroups per CU of the streaming kernel, by [row tiles][sub-tiles]
  // workspace (owned)
  void* xq;
  void* xs;
  float* part;
  uint32_t* cnt;
  size_t xq_bytes, xs_bytes, part_bytes, cnt_bytes;
  int staged_R;   // rows of the operands last staged (-1: none)
};

static const uint32_t HANDLE_MAGIC = 0x51474D31u;  // "QGM1"
static const uint32_t SEQ_MAGIC = 0x51475331u;     // "QGS1"

namespace {

struct Plan {
  int path;
  int RT, NT;
  int64_t T, I, P;
  int kernels;
  size_t part_bytes, cnt_bytes, ws_bytes;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_shape(int64_t N, int64_t K) {
  if (N < 1 || K < 256 || K % 256 != 0) return false;
  if (N > (int64_t(1) << 40) || K > (int64_t(1) << 30)) return false;
  // the kernels address each region with 32-bit offsets
  if (quant_region_bytes(N, K) >= (int64_t(1) << 31)) return false;
  if ((K / 256) * 8192 * 4 >= (int64_t(1) << 31)) return false;
  return true;
}

bool valid_handle(const qgemm_handle* h) { return h && h->magic == HANDLE_MAGIC; }

// Matrix-core plan: 16-row tiles, NT 16-output sub-tiles per wave, 4 waves per
// workgroup, and as many workgroups as stay resident on the device (each gets
// an equal share of the (tile, block) steps), but never fewer than two steps
// per workgroup.
Plan plan_stream(int64_t NS, int64_t KB, int R, int cus, const int occ[5][5]) {
  Plan p{};
  p.path = QGEMM_PATH_MFMA;
  p.RT = (R + 15) / 16;
  p.NT = (p.RT <= 2) ? 2 : 1;
  p.T = (NS + 4 * p.NT - 1) / (4 * p.NT);
  p.I = p.T * KB;
  int64_t resident = (int64_t)cus * std::max(1, occ[p.RT][p.NT]);
  p.P = std::max<int64_t>(1, std::min(resident, p.I / 2));
  p.kernels = 1;
  p.part_bytes = (size_t)(2 * p.P) * 4 * p.NT * p.RT * 256 * 4;
  p.cnt_bytes = (size_t)p.T * 4;
  p.ws_bytes = (size_t)p.RT * KB * 8192 + (size_t)p.RT * KB * 512 + p.part_bytes + p.cnt_bytes;
  return p;
}

int make_plan(const qgemm_handle* h, int R, int path, Plan* out) {
  if (path == QGEMM_PATH_VALU) return QGEMM_EPATH;
  if (path != QGEMM_PATH_AUTO && path != QGEMM_PATH_MFMA) return QGEMM_EINVAL;
  *out = plan_stream(h->NS, h->KB, R, h->cus, h->occ);
  return QGEMM_OK;
}

int stage_impl(qgemm_handle* h, const void* x, int R, hipStream_t st) {
  int RT = (R + 15) / 16;
  hipError_t e = launch_xprep(reinterpret_cast<const uint16_t*>(x), h->xq, h->xs, R, h->K, RT, st);
  if (e != hipSuccess) return QGEMM_EHIP;
  h->staged_R = R;
  return QGEMM_OK;
}

int multiply_impl(qgemm_handle* h, float* y, int R, int path, hipStream_t st) {
  Plan p;
  int rc = make_plan(h, R, path, &p);
  if (rc) return rc;
  StreamArgs a{};
  a.packed = h->packed;
  a.hdr_off = quant_region_bytes(h->N, h->K);
  a.quant_bytes = (uint32_t)a.hdr_off;
  a.hdr_bytes = (uint32_t)(packed_bytes(h->N, h->K) - a.hdr_off);
  a.xq = h->xq;
  a.xs = h->xs;
  a.y = y;
  a.part = h->part;
  a.cnt = h->cnt;
  a.N = h->N;
  a.NS = h->NS;
  a.KB = (int)h->KB;
  a.R = R;
  a.T = p.T;
  a.I = p.I;
  a.P = p.P;
  a.RT = p.RT;
  a.NT = p.NT;
  return launch_stream(a, st) == hipSuccess ? QGEMM_OK : QGEMM_EHIP;
}

int run_impl(qgemm_handle* h, const void* x, float* y, int R, int path, hipStream_t st) {
  Plan p;
  int rc = make_plan(h, R, path, &p);
  if (rc) return rc;
  rc = stage_impl(h, x, R, st);
  if (rc) return rc;
  return multiply_impl(h, y, R, path, st);
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
  for (int rt = 0; rt < 5; ++rt)
    for (int nt = 0; nt < 5; ++nt) h->occ[rt][nt] = (rt && nt) ? stream_occupancy(rt, nt) : 0;
  int rt_max = (max_R + 15) / 16;
  h->xq_bytes = (size_t)rt_max * h->KB * 8192;
  h->xs_bytes = (size_t)rt_max * h->KB * 512;
  size_t part = 0, cnt = 0;
  for (int R = 1; R <= max_R; ++R) {
    Plan p = plan_stream(h->NS, h->KB, R, cus, h->occ);
    part = std::max(part, p.part_bytes);
    cnt = std::max(cnt, p.cnt_bytes);
  }
  h->part_bytes = part;
  h->cnt_bytes = cnt;
  h->staged_R = -1;
  bool ok = hipMalloc(&h->xq, h->xq_bytes) == hipSuccess && hipMalloc(&h->xs, h->xs_bytes) == hipSuccess;
  if (ok && part) ok = hipMalloc(reinterpret_cast<void**>(&h->part), part) == hipSuccess;
  if (ok && cnt) ok = hipMalloc(reinterpret_cast<void**>(&h->cnt), cnt) == hipSuccess &&
                      hipMemset(h->cnt, 0, cnt) == hipSuccess && hipDeviceSynchronize() == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    if (h->xq) (void)hipFree(h->xq);
    if (h->xs) (void)hipFree(h->xs);
    if (h->part) (void)hipFree(h->part);
    if (h->cnt) (void)hipFree(h->cnt);
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

int qgemm_stage(qgemm_t h, const void* x_bf16, int R, void* stream) {
  if (!valid_handle(h)) return QGEMM_EINVAL;
  if (R < 0 || R > h->max_R) return QGEMM_ERANGE_R;
  if (R == 0) return QGEMM_OK;
  if (!x_bf16) return QGEMM_EINVAL;
  if (!aligned16(x_bf16)) return QGEMM_EALIGN;
  return stage_impl(h, x_bf16, R, reinterpret_cast<hipStream_t>(stream));
}

int qgemm_multiply(qgemm_t h, float* y, int R, int path, void* stream) {
  if (!valid_handle(h)) return QGEMM_EINVAL;
  if (R < 0 || R > h->max_R) return QGEMM_ERANGE_R;
  if (path < QGEMM_PATH_AUTO || path > QGEMM_PATH_MFMA) return QGEMM_EINVAL;
  if (R == 0) return QGEMM_OK;
  if (R != h->staged_R) return QGEMM_ERANGE_R;
  if (!y) return QGEMM_EINVAL;
  if (!aligned16(y)) return QGEMM_EALIGN;
  return multiply_impl(h, y, R, path, reinterpret_cast<hipStream_t>(stream));
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
  info->row_tiles = p.RT;
  info->subtiles_per_wave = p.NT;
  info->tiles = p.T;
  info->workgroups = p.P;
  info->steps = p.I;
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
  if (h->cnt) (void)hipFree(h->cnt);
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
