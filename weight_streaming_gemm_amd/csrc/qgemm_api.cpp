// qgemm_api.cpp — host side of the C ABI: argument validation, the
// R-dependent launch plan, workspace ownership and the graph-captured pass.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/qgemm.h"
#include "layout.h"
#include "pass_sched.h"
#include "qgemm_internal.h"

using namespace qg;
static_assert(MAX_ROWS == QGEMM_MAX_R, "row limit of the kernels and of the ABI");

struct qgemm_handle {
  uint32_t magic;
  const uint8_t* packed;
  int64_t N, K, KB, NS;
  int max_R;
  int cus;
  int occ[5];     // resident workgroups per CU of the streaming kernel, by row tiles
  // workspace (owned)
  float* part;
  uint32_t* cnt;
  size_t part_bytes, cnt_bytes;
  void* tiled_ws;           // the row-tiled path's image and partials (max_R >= QGEMM_TILED_MIN_R)
  size_t tiled_ws_bytes;
};

static const uint32_t HANDLE_MAGIC = 0x51474D32u;  // "QGM2"
static const uint32_t SEQ_MAGIC = 0x51475332u;     // "QGS2"

namespace {

struct Plan {
  int path;
  int RT, NT, NW, nwn, aligned, msum;
  int64_t S, kbv, treal;   // K in S chunks of kbv blocks (S = 1: kbv = KB) over treal output tiles
  int64_t T, I, V, P;
  size_t part_bytes, cnt_bytes;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_shape(int64_t N, int64_t K) {
  if (N < 1 || K < 256 || K % 256 != 0) return false;
  if (N > (int64_t(1) << 40) || K > (int64_t(1) << 30)) return false;
  // the kernels address each region, and x, with 32-bit offsets
  if (quant_region_bytes(N, K) >= (int64_t(1) << 31)) return false;
  if ((int64_t)QGEMM_MAX_R * K * 2 >= (int64_t(1) << 31)) return false;
  return true;
}

bool valid_handle(const qgemm_handle* h) { return h && h->magic == HANDLE_MAGIC; }

// R rows = agents of D + 1 rows each (current token and D drafts)
bool verify_args_ok(int R, const int32_t* drafts, int D, const int32_t* tokens, const int32_t* n_new) {
  return D >= 0 && R % (D + 1) == 0 && (D == 0 || drafts) && tokens && n_new;
}

// The min term from staged sub-block sums costs work per staged block and saves
// seven products per step: taken when a range has at least 4 steps per block
// (and the sums fit in LDS).
void choose_msum(Plan& p, int64_t KB, int R) {
  const int64_t steps = p.aligned ? ((p.T + p.V - 1) / p.V) * KB : (p.I + p.V - 1) / p.V;
  const int64_t slots = std::min(steps, KB);
  p.msum = steps >= 4 * slots && slots <= x_slot_capacity(R, p.RT, p.NT, p.NW, true);
}

// Matrix-core plan for one GEMM: 16-row tiles, NW waves per workgroup in an
// nwn x (NW / nwn) grid, tiles of nwn * NT 16-output sub-tiles, one workgroup
// per CU, one range of (tile, block) steps per workgroup.  V = P ranges: as
// many as stay resident (at most P_cap), fewer if there are fewer steps.  A
// range's activations must fit the workgroup's LDS: nwn is the smallest wave
// grid width for which they do (wider tiles mean fewer steps per range); if
// none does, the widest grid runs ranges of at most cap steps in several rounds.
//
// valu: the same schedule for the vector-unit kernel (R <= VALU_MAX_R, one row
// tile), which always takes the min term from the staged sub-block sums.
Plan plan_stream(int64_t NS, int64_t KB, int R, int cus, const int occ[5], int64_t P_cap = 0,
                 bool valu = false) {
  Plan p{};
  p.path = valu ? QGEMM_PATH_VALU : QGEMM_PATH_MFMA;
  p.S = 1;
  p.kbv = KB;
  p.RT = (R + 15) / 16;
  p.NW = waves_for(p.RT);
  p.NT = subtiles_for(p.RT);
  int64_t resident = (int64_t)cus * std::max(1, occ[p.RT]);
  if (P_cap > 0) resident = std::min(resident, P_cap);
  const int64_t cap = x_slot_capacity(R, p.RT, p.NT, p.NW, valu);
  auto min_term = [&](int64_t kb) {
    if (valu)
      p.msum = 1;
    else
      choose_msum(p, kb, R);
  };
  // Ranges of whole tiles need no partial sums across workgroups (whose
  // exchange costs a few memory round trips at the end of a range, worth about
  // FIXUP_STEPS steps); they are taken when every workgroup gets a tile, a
  // whole tile row of activations fits in LDS, and the uneven split costs less.
  constexpr int64_t FIXUP_STEPS = 32;
  const int64_t T1 = (NS + p.NT - 1) / p.NT;
  if (KB <= cap && T1 >= resident) {
    const int64_t V = resident;
    if (((T1 + V - 1) / V) * KB <= (T1 * KB + V - 1) / V + FIXUP_STEPS) {
      p.nwn = 1;
      p.aligned = 1;
      p.T = T1;
      p.I = T1 * KB;
      p.V = p.P = V;
      p.treal = p.T;
      p.part_bytes = 0;
      p.cnt_bytes = (size_t)p.T * 4;
      min_term(KB);
      return p;
    }
  }
  bool one_round = false;
  for (int nwn = 1; nwn <= p.NW; nwn *= 2) {
    if (p.NW % nwn) break;
    p.nwn = nwn;
    p.T = (NS + (int64_t)nwn * p.NT - 1) / ((int64_t)nwn * p.NT);
    p.I = p.T * KB;
    p.V = std::max<int64_t>(1, std::min(resident, p.I));
    if (std::min((p.I + p.V - 1) / p.V, KB) <= cap) { one_round = true; break; }
  }
  if (!one_round) {
    // No wave grid fits a range's activations in one round: K in S chunks of
    // kbv blocks (the largest divisor of KB that fits), resident / S ranges of
    // whole tiles per chunk; each chunk of a tile leaves a partial result.
    int64_t kc = std::max<int64_t>(1, std::min(cap, KB));
    while (KB % kc) --kc;
    p.nwn = 1;
    p.aligned = 1;
    p.S = KB / kc;
    p.kbv = kc;
    p.treal = T1;
    // (a range's tiles arrive one thread each: at most NW * 64 tiles per range)
    const int64_t vc = std::max((T1 + p.NW * 64 - 1) / (p.NW * 64),
                                std::min(T1, std::max<int64_t>(1, resident / p.S)));
    p.T = p.S * T1;
    p.I = p.T * kc;
    p.V = p.P = p.S * vc;
    p.part_bytes = (size_t)p.T * partial_slot_bytes(p.RT, p.NT, 1);
    p.cnt_bytes = (size_t)T1 * 4;
    min_term(kc);
    return p;
  }
  p.P = p.V;
  p.treal = p.T;
  p.part_bytes = (size_t)(2 * p.V) * partial_slot_bytes(p.RT, p.NT, p.nwn);
  p.cnt_bytes = (size_t)p.T * 4;
  min_term(KB);
  return p;
}

// the kernel's schedule arithmetic is 32-bit: (V + 1) * I must stay below 2^31
bool plan_fits(const Plan& p) { return (p.V + 1) * (p.I + 1) < (int64_t(1) << 31); }

// The R-dependent choice: the vector-unit kernel for R <= VALU_AUTO_MAX_R (the
// measured crossover: below it the vector-unit kernel streams faster), the
// matrix-core kernel above.
// The row-tiled kernel (measured per matrix over R = 12..64 on one layer): from
// QGEMM_TILED_MIN_R rows on for wide matrices (N >= 32768: gate|up, the output
// head; there its 32-row grid with two workgroups per CU beats the streaming
// kernel's re-staged activations), from 48 rows on for matrices of at least 2^26
// weights (down as well), and at QGEMM_MAX_R rows for all.
bool auto_tiled(const qgemm_handle* h, int R) {
  if (h->max_R < QGEMM_TILED_MIN_R || R < QGEMM_TILED_MIN_R) return false;
  return R >= QGEMM_MAX_R || h->N >= 32768 || (R >= 48 && h->N * h->K >= (int64_t(1) << 26));
}

int make_plan(const qgemm_handle* h, int R, int path, Plan* out) {
  if (path != QGEMM_PATH_AUTO && path != QGEMM_PATH_MFMA && path != QGEMM_PATH_VALU && path != QGEMM_PATH_TILED)
    return QGEMM_EINVAL;
  if (path == QGEMM_PATH_VALU && R > VALU_MAX_R) return QGEMM_EPATH;
  if (path == QGEMM_PATH_TILED && h->max_R < QGEMM_TILED_MIN_R) return QGEMM_EPATH;
  if (path == QGEMM_PATH_TILED || (path == QGEMM_PATH_AUTO && auto_tiled(h, R))) {
    *out = Plan{};
    out->path = QGEMM_PATH_TILED;
    return QGEMM_OK;
  }
  const bool valu = path == QGEMM_PATH_VALU || (path == QGEMM_PATH_AUTO && R <= VALU_AUTO_MAX_R);
  *out = plan_stream(h->NS, h->KB, R, h->cus, h->occ, 0, valu);
  return plan_fits(*out) ? QGEMM_OK : QGEMM_ESHAPE;
}

GemmDesc make_desc(const qgemm_handle* h, const void* x, float* y, const Plan& p) {
  GemmDesc d{};
  d.packed = h->packed;
  d.x = reinterpret_cast<const uint16_t*>(x);
  d.y = y;
  d.quant_bytes = (uint32_t)quant_region_bytes(h->N, h->K);
  d.hdr_bytes = (uint32_t)(packed_bytes(h->N, h->K) - d.quant_bytes);
  d.N = (int32_t)h->N;
  d.NS = (int32_t)h->NS;
  d.nwn = (int32_t)p.nwn;
  d.T = (int32_t)p.T;
  d.I = (int32_t)p.I;
  d.V = (int32_t)p.V;
  d.aligned = p.aligned;
  d.KB = (int32_t)p.kbv;                 // blocks per tile of the step order (a chunk's)
  d.S = (int32_t)p.S;
  d.kbr = (int32_t)h->KB;
  d.treal = (int32_t)p.treal;
  return d;
}

int run_impl(qgemm_handle* h, const void* x, float* y, int R, int path, hipStream_t st) {
  Plan p;
  int rc = make_plan(h, R, path, &p);
  if (rc) return rc;
  if (p.path == QGEMM_PATH_TILED) {
    const PrefillPlan tp = prefill_plan(h->N, h->K, R, h->cus);
    if (tp.ws_bytes > h->tiled_ws_bytes) return QGEMM_EHIP;      // sized at create for every R <= max_R
    return launch_prefill(h->packed, h->N, h->K, x, y, R, tp, h->tiled_ws, st) == hipSuccess ? QGEMM_OK : QGEMM_EHIP;
  }
  StreamArgs a{};
  a.d0 = make_desc(h, x, y, p);
  a.part = h->part;
  a.cnt = h->cnt;
  a.R = R;
  a.P = (int32_t)p.P;
  a.RT = p.RT;
  a.NT = p.NT;
  a.NW = p.NW;
  a.msum = p.msum;
  a.valu = p.path == QGEMM_PATH_VALU;
  return launch_stream(a, st) == hipSuccess ? QGEMM_OK : QGEMM_EHIP;
}

int device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QGEMM_EHIP;
  if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || *cus <= 0)
    return QGEMM_EHIP;
  return QGEMM_OK;
}

void fill_occupancy(int occ[5]) {
  occ[0] = 0;
  for (int rt = 1; rt < 5; ++rt) occ[rt] = stream_occupancy(rt, subtiles_for(rt), waves_for(rt));
}

// Per-device facts for qgemm_run_static, gathered on its first call on a device
// (with that device current) and kept: compute units, resident workgroups of
// the streaming kernel, and the device address of the fixed scratch area.
struct StaticDevice {
  bool ready;
  int cus;
  int occ[5];
  void* scratch;
};

int static_device(const StaticDevice** out) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static StaticDevice table[MAX_DEVICES] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return QGEMM_EHIP;
  std::lock_guard<std::mutex> lock(mu);
  StaticDevice& d = table[dev];
  if (!d.ready) {
    if (device_cus(&d.cus) != QGEMM_OK) return QGEMM_EHIP;
    fill_occupancy(d.occ);
    if (static_scratch_address(&d.scratch) != hipSuccess || !d.scratch) return QGEMM_EHIP;
    d.ready = true;
  }
  *out = &d;
  return QGEMM_OK;
}

}  // namespace

extern "C" {

int qgemm_read_probe(const void* buf, uint64_t bytes, void* sink, void* stream) {
  if (!buf || !sink || bytes % 16 != 0 || bytes >= (1ull << 40)) return QGEMM_EINVAL;
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 16 != 0) return QGEMM_EALIGN;
  int cus = 0;
  if (const int rc = device_cus(&cus)) return rc;
  if (bytes == 0) return QGEMM_OK;
  return launch_read_probe(buf, bytes, sink, cus, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? QGEMM_OK
                                                                                                       : QGEMM_EHIP;
}

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
    case QGEMM_ESCRATCH: return "the run needs more than the fixed scratch area of qgemm_run_static";
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
  if (device_cus(&h->cus) != QGEMM_OK) {
    delete h;
    return QGEMM_EHIP;
  }
  fill_occupancy(h->occ);
  size_t part = 0, cnt = 0;
  for (int R = 1; R <= max_R; ++R)
    for (int valu = 0; valu < (R <= VALU_MAX_R ? 2 : 1); ++valu) {
      Plan p = plan_stream(h->NS, h->KB, R, h->cus, h->occ, 0, valu != 0);
      if (!plan_fits(p)) {
        delete h;
        return QGEMM_ESHAPE;
      }
      part = std::max(part, p.part_bytes);
      cnt = std::max(cnt, p.cnt_bytes);
    }
  part = std::max<size_t>(part, 256);
  h->part_bytes = part;
  h->cnt_bytes = cnt;
  size_t tiled = 0;
  if (max_R >= QGEMM_TILED_MIN_R)
    for (int R = 1; R <= max_R; ++R) tiled = std::max(tiled, prefill_plan(N, K, R, h->cus).ws_bytes);
  h->tiled_ws_bytes = tiled;
  bool ok = hipMalloc(reinterpret_cast<void**>(&h->part), part) == hipSuccess &&
            hipMalloc(reinterpret_cast<void**>(&h->cnt), cnt) == hipSuccess &&
            (tiled == 0 || hipMalloc(&h->tiled_ws, tiled) == hipSuccess) &&
            hipMemset(h->cnt, 0, cnt) == hipSuccess && hipDeviceSynchronize() == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    if (h->part) (void)hipFree(h->part);
    if (h->cnt) (void)hipFree(h->cnt);
    if (h->tiled_ws) (void)hipFree(h->tiled_ws);
    delete h;
    return QGEMM_ENOMEM;
  }
  *out = h;
  return QGEMM_OK;
}

int qgemm_run_path(qgemm_t h, const void* x_bf16, float* y, int R, int path, void* stream) {
  if (!valid_handle(h)) return QGEMM_EINVAL;
  if (R < 0 || R > h->max_R) return QGEMM_ERANGE_R;
  if (path < QGEMM_PATH_AUTO || path > QGEMM_PATH_TILED) return QGEMM_EINVAL;
  if (R == 0) return QGEMM_OK;
  if (!x_bf16 || !y) return QGEMM_EINVAL;
  if (!aligned16(x_bf16) || !aligned16(y)) return QGEMM_EALIGN;
  return run_impl(h, x_bf16, y, R, path, reinterpret_cast<hipStream_t>(stream));
}

int qgemm_run(qgemm_t h, const void* x_bf16, float* y, int R, void* stream) {
  return qgemm_run_path(h, x_bf16, y, R, QGEMM_PATH_AUTO, stream);
}

int qgemm_run_static(const void* packed_dev, int64_t N, int64_t K, const void* x_bf16, float* y, int R,
                     void* stream) {
  if (!packed_dev) return QGEMM_EINVAL;
  if (!valid_shape(N, K)) return QGEMM_ESHAPE;
  if (R < 0 || R > QGEMM_MAX_R) return QGEMM_ERANGE_R;
  if (R == 0) return QGEMM_OK;
  if (!x_bf16 || !y) return QGEMM_EINVAL;
  if (!aligned16(packed_dev) || !aligned16(x_bf16) || !aligned16(y)) return QGEMM_EALIGN;
  const StaticDevice* sd = nullptr;
  if (static_device(&sd) != QGEMM_OK) return QGEMM_EHIP;
  // a handle on the stack: borrowed weights, no workspace of its own
  qgemm_handle h{};
  h.magic = HANDLE_MAGIC;
  h.packed = reinterpret_cast<const uint8_t*>(packed_dev);
  h.N = N;
  h.K = K;
  h.KB = K / 256;
  h.NS = padded_n(N) / 16;
  h.max_R = R;
  h.cus = sd->cus;
  const Plan p = plan_stream(h.NS, h.KB, R, sd->cus, sd->occ);
  if (!plan_fits(p)) return QGEMM_ESHAPE;
  const size_t cnt_bytes = (p.cnt_bytes + 255) / 256 * 256;
  if (cnt_bytes + p.part_bytes > STATIC_SCRATCH_BYTES) return QGEMM_ESCRATCH;
  uint8_t* const base = reinterpret_cast<uint8_t*>(sd->scratch);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // the previous call's counters may not be zero if it did not complete: clear them
  if (launch_zero_words(reinterpret_cast<uint32_t*>(base), (int64_t)(cnt_bytes / 4), st) != hipSuccess)
    return QGEMM_EHIP;
  StreamArgs a{};
  a.d0 = make_desc(&h, x_bf16, y, p);
  a.part = reinterpret_cast<float*>(base + cnt_bytes);
  a.cnt = reinterpret_cast<uint32_t*>(base);
  a.R = R;
  a.P = (int32_t)p.P;
  a.RT = p.RT;
  a.NT = p.NT;
  a.NW = p.NW;
  a.msum = p.msum;
  a.valu = 0;
  return launch_stream(a, st) == hipSuccess ? QGEMM_OK : QGEMM_EHIP;
}

int qgemm_prefill_workspace_size(qgemm_t h, int R, size_t* bytes) {
  if (!valid_handle(h) || !bytes) return QGEMM_EINVAL;
  if (R < 0 || R > QGEMM_MAX_PREFILL_R) return QGEMM_ERANGE_R;
  if (R == 0) {
    *bytes = 0;
    return QGEMM_OK;
  }
  const PrefillPlan p = prefill_plan(h->N, h->K, R, h->cus);
  if (p.img_bytes >= (size_t(1) << 31)) return QGEMM_ERANGE_R;
  *bytes = p.ws_bytes;
  return QGEMM_OK;
}

int qgemm_run_prefill(qgemm_t h, const void* x_bf16, float* y, int R, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (!valid_handle(h)) return QGEMM_EINVAL;
  if (R < 0 || R > QGEMM_MAX_PREFILL_R) return QGEMM_ERANGE_R;
  if ((int64_t)R * h->K * 2 >= (int64_t(1) << 31)) return QGEMM_ERANGE_R;   // x is addressed with 32-bit offsets
  if (R == 0) return QGEMM_OK;
  if (!x_bf16 || !y) return QGEMM_EINVAL;
  if (!aligned16(x_bf16) || !aligned16(y)) return QGEMM_EALIGN;
  const PrefillPlan p = prefill_plan(h->N, h->K, R, h->cus);
  if (p.img_bytes >= (size_t(1) << 31)) return QGEMM_ERANGE_R;     // the image is addressed with 32-bit offsets
  if (!workspace || workspace_bytes < p.ws_bytes) return QGEMM_EINVAL;
  if (!aligned16(workspace)) return QGEMM_EALIGN;
  return launch_prefill(h->packed, h->N, h->K, x_bf16, y, R, p, workspace, reinterpret_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? QGEMM_OK
             : QGEMM_EHIP;
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

int qgemm_argmax_workspace_size(int R, int64_t N, size_t* bytes) {
  if (!bytes) return QGEMM_EINVAL;
  if (R < 0 || R > QGEMM_MAX_R) return QGEMM_ERANGE_R;
  if (N < 1 || N > INT32_MAX) return QGEMM_ESHAPE;
  *bytes = argmax_ws_bytes(R, N);
  return QGEMM_OK;
}

int qgemm_argmax_rows_ws(const float* y, int R, int64_t N, int32_t* idx, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (R < 0 || R > QGEMM_MAX_R) return QGEMM_ERANGE_R;
  if (N < 1 || N > INT32_MAX) return QGEMM_ESHAPE;
  if (R == 0) return QGEMM_OK;
  if (!y || !idx || !workspace || workspace_bytes < argmax_ws_bytes(R, N)) return QGEMM_EINVAL;
  if (!aligned16(workspace)) return QGEMM_EALIGN;
  hipError_t e = launch_argmax_split(y, R, N, idx, workspace, nullptr, 0, nullptr, nullptr,
                                     reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? QGEMM_OK : QGEMM_EHIP;
}

int qgemm_verify_greedy(const int32_t* argmax_idx, int R, const int32_t* drafts, int drafts_per_agent,
                        int32_t* tokens, int32_t* n_new, void* stream) {
  if (R < 0 || R > QGEMM_MAX_R) return QGEMM_ERANGE_R;
  if (!verify_args_ok(R, drafts, drafts_per_agent, tokens, n_new)) return QGEMM_EINVAL;
  if (R == 0) return QGEMM_OK;
  if (!argmax_idx) return QGEMM_EINVAL;
  hipError_t e = launch_verify(argmax_idx, R, drafts, drafts_per_agent, tokens, n_new,
                               reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? QGEMM_OK : QGEMM_EHIP;
}

int qgemm_query(qgemm_t h, int R, int path, qgemm_info* info) {
  if (!valid_handle(h) || !info) return QGEMM_EINVAL;
  if (R < 1 || R > h->max_R) return QGEMM_ERANGE_R;
  Plan p;
  int rc = make_plan(h, R, path, &p);
  if (rc) return rc;
  if (p.path == QGEMM_PATH_TILED) {
    const PrefillPlan tp = prefill_plan(h->N, h->K, R, h->cus);
    *info = qgemm_info{};
    info->path = QGEMM_PATH_TILED;
    info->tiles = tp.mt * tp.nt;
    info->workgroups = tp.mt * tp.nt * tp.S;
    info->kernels = tp.S > 1 ? 3 : 2;
    info->k_chunks = (int)tp.S;
    info->workspace_bytes = tp.ws_bytes;
    info->min_term_sums = 1;
    return QGEMM_OK;
  }
  info->path = p.path;
  info->row_tiles = p.path == QGEMM_PATH_VALU ? 0 : p.RT;
  info->subtiles_per_wave = p.NT;
  info->tiles = p.T;
  info->workgroups = p.P;
  info->steps = p.I;
  info->kernels = 1;
  info->workspace_bytes = p.part_bytes + p.cnt_bytes;
  info->ranges = p.V;
  info->waves_per_workgroup = p.NW;
  info->wave_columns = p.nwn;
  info->whole_tile_ranges = p.aligned;
  info->k_chunks = (int)p.S;
  info->min_term_sums = p.msum;
  return QGEMM_OK;
}

int qgemm_destroy(qgemm_t h) {
  if (!h) return QGEMM_OK;
  if (!valid_handle(h)) return QGEMM_EINVAL;
  (void)hipDeviceSynchronize();
  if (h->part) (void)hipFree(h->part);
  if (h->cnt) (void)hipFree(h->cnt);
  if (h->tiled_ws) (void)hipFree(h->tiled_ws);
  h->magic = 0;
  delete h;
  return QGEMM_OK;
}

}  // extern "C"

// ---- full weight pass --------------------------------------------------------

struct SeqKey {
  int R;
  std::vector<uintptr_t> ptrs;
  bool operator<(const SeqKey& o) const {
    if (R != o.R) return R < o.R;
    return ptrs < o.ptrs;
  }
};

struct qgemm_seq {
  uint32_t magic;
  uint32_t flags;
  std::vector<qgemm_handle*> hs;
  hipStream_t cap;                                 // capture stream (graph mode)
  std::map<SeqKey, hipGraphExec_t> graphs;         // per (R, pointer set) (graph mode)
  int cus;
  // persistent mode (pass.hip): workspace shared by the GEMMs of a launch
  float* part;       // chunk partial tiles
  uint32_t* cnt;     // per-sub-tile chunk arrival counters
  uint32_t* bar;     // barrier counters
  uint32_t* err;
  size_t part_bytes, cnt_bytes;
  std::map<SeqKey, PassGemm*> descs;   // device descriptor tables per (R, pointer set)
  std::map<int, PassWave*> waves;      // device wave tables per R
  std::vector<char> gated;             // GEMM g waits only for the producers of its inputs
  std::map<int, uint64_t*> masks;      // device bitmasks of those producers per R (gated GEMMs)
  void* am_ws;       // argmax (and verification) workspace for the last GEMM's output
  int max_R;
};

namespace {

// K chunks of one GEMM in the persistent pass at R rows: the fewest (dividing
// the blocks of K, at most pass_max_chunks and at most one per workgroup) whose
// activations fit the kernel's LDS area at R's row tiles; 0 when none does.
int pass_chunks_of(int64_t KB, int R, int P) {
  if (KB > INT32_MAX || R < 1 || R > PASS_MAX_R) return 0;
  return pass_chunks((int)KB, R, P, pass_x_area(pass_row_tiles(R)), pass_max_chunks(pass_row_tiles(R)));
}

// The GEMMs' chunking and workspace needs at R rows; false if a GEMM cannot run
bool pass_sizes(const qgemm_seq* s, int R, size_t* part, size_t* cnt) {
  *part = *cnt = 0;
  if (R < 1 || R > PASS_MAX_R) return false;
  for (const qgemm_handle* h : s->hs) {
    const int S = pass_chunks_of(h->KB, R, s->cus);
    if (S == 0) return false;
    if (S > 1) {
      *part = std::max(*part, (size_t)S * (size_t)h->NS * 1024 * pass_row_tiles(R));
      *cnt = std::max(*cnt, (size_t)h->NS * 4);
    }
  }
  *part *= 2;        // halves for GEMMs of even and odd index
  *cnt *= 2;
  return true;
}

// Gated inputs: GEMM g (g > 0) reads, for input column j, only the previous
// GEMM's outputs j and K + j (a fused gate|up of 2 K outputs through an
// element-wise gate).  Taken where the shapes say so, never for two GEMMs in a
// row (so at most two GEMMs are in flight), and for at most PASS_MAX_GATED_P
// workgroups.
std::vector<char> gated_gemms(const qgemm_seq* s) {
  std::vector<char> v(s->hs.size(), 0);
  if (!(s->flags & QGEMM_SEQ_GATED_INPUTS) || s->cus > PASS_MAX_GATED_P) return v;
  for (size_t g = 1; g < s->hs.size(); ++g)
    v[g] = s->hs[g - 1]->N == 2 * s->hs[g]->K && s->hs[g]->K % TILE_N == 0 && !v[g - 1];
  return v;
}

// per gated GEMM and chunk, PASS_MASK_WORDS words: a bitmask of the workgroups
// whose units of the previous GEMM hold the outputs the chunk reads, then the
// chunk counter's target; offsets[g] indexes the GEMM's first chunk (in words),
// -1 if it waits for every workgroup
std::vector<uint64_t> gated_masks(const qgemm_seq* s, int R, std::vector<int64_t>* offsets) {
  std::vector<uint64_t> m;
  offsets->assign(s->hs.size(), -1);
  const int P = s->cus;
  uint64_t target[PASS_MAX_CHUNKS] = {};                            // per chunk index, over the launch
  for (size_t g = 1; g < s->hs.size(); ++g) {
    if (!s->gated[g]) continue;
    const qgemm_handle* prev = s->hs[g - 1];
    const qgemm_handle* cur = s->hs[g];
    const int Sp = pass_chunks_of(prev->KB, R, P), Sc = pass_chunks_of(cur->KB, R, P);
    const int rot_p = (int)(((g - 1) * 37) % (size_t)P);
    (*offsets)[g] = (int64_t)m.size();
    for (int c = 0; c < Sc; ++c) {
      uint64_t w[PASS_MASK_WORDS] = {};
      pass_gated_mask(c, (int)(cur->KB / Sc), (int)(cur->K / TILE_N), P, (int)prev->NS, Sp, rot_p, w);
      // the chunk counter's value once these workgroups are through (the counter
      // keeps counting over the launch's gated GEMMs)
      target[c] += (uint64_t)(__builtin_popcountll(w[0]) + __builtin_popcountll(w[1]) +
                              __builtin_popcountll(w[2]) + __builtin_popcountll(w[3]));
      w[4] = target[c];
      m.insert(m.end(), w, w + PASS_MASK_WORDS);
    }
  }
  return m;
}

// the descriptor table of one run (the GEMMs' weights, activations, outputs and
// chunking at R rows); rot spreads the longer unit runs over the workgroups
std::vector<PassGemm> pass_descs(const qgemm_seq* s, int R, const void* const* xs, float* const* ys,
                                  const uint64_t* masks_dev, const std::vector<int64_t>& mask_off) {
  std::vector<PassGemm> t(s->hs.size());
  for (size_t g = 0; g < s->hs.size(); ++g) {
    const qgemm_handle* h = s->hs[g];
    PassGemm& d = t[g];
    const int64_t qb = quant_region_bytes(h->N, h->K);
    d.qbase = h->packed;
    d.hbase = h->packed + qb;
    d.qbytes = (uint32_t)qb;
    d.hbytes = (uint32_t)(packed_bytes(h->N, h->K) - qb);
    d.x = reinterpret_cast<const uint16_t*>(xs[g]);
    d.y = ys[g];
    d.N = (int32_t)h->N;
    d.NS = (int32_t)h->NS;
    d.KB = (int32_t)h->KB;
    d.S = pass_chunks_of(h->KB, R, s->cus);
    d.kbc = (int32_t)(h->KB / d.S);
    d.rot = (int32_t)((g * 37) % (size_t)s->cus);
    d.masks = mask_off[g] >= 0 ? masks_dev + mask_off[g] : nullptr;
  }
  return t;
}

// every compute wave's share of every GEMM (pass_sched.h), [G][P][PASS_NC]
std::vector<PassWave> pass_waves(const std::vector<PassGemm>& t, int P) {
  const int G = (int)t.size();
  std::vector<PassWave> v((size_t)G * P * PASS_NC);
  for (int g = 0; g < G; ++g) {
    const PassGemm& d = t[g];
    for (int p = 0; p < P; ++p)
      for (int w = 0; w < PASS_NC; ++w) {
        PassWave& e = v[((size_t)g * P + p) * PASS_NC + w];
        pass_wave_share(p, w, PASS_NC, P, d.NS, d.KB, d.S, d.kbc, d.rot, &e.count, &e.step0, &e.jj0);
        int c, ns0, ns1;
        pass_units(p, d.S, P, d.NS, d.rot, &c, &ns0, &ns1);
        e.xblk = ns1 > ns0 ? d.kbc : 0;
      }
  }
  // next: the first later GEMM where the wave has steps
  for (int p = 0; p < P; ++p)
    for (int w = 0; w < PASS_NC; ++w) {
      int next = G;
      for (int g = G - 1; g >= 0; --g) {
        PassWave& e = v[((size_t)g * P + p) * PASS_NC + w];
        e.next = next;
        if (e.count > 0) next = g;
      }
    }
  return v;
}

// Cached graphs and descriptor tables per (R, pointer set): at most this many
// of each; a run that needs another waits for the device and drops them all
// (a graph or table may still be in use by work in flight).
constexpr size_t SEQ_CACHE_MAX = 64;

void seq_drop_graphs(qgemm_seq* s) {
  (void)hipDeviceSynchronize();
  for (auto& kv : s->graphs) (void)hipGraphExecDestroy(kv.second);
  s->graphs.clear();
}

void seq_drop_descs(qgemm_seq* s) {
  (void)hipDeviceSynchronize();
  for (auto& kv : s->descs) (void)hipFree(kv.second);
  s->descs.clear();
}

void seq_free(qgemm_seq* s) {
  for (auto& kv : s->graphs) (void)hipGraphExecDestroy(kv.second);
  if (s->cap) (void)hipStreamDestroy(s->cap);
  for (auto& kv : s->descs) (void)hipFree(kv.second);
  for (auto& kv : s->waves) (void)hipFree(kv.second);
  for (auto& kv : s->masks) (void)hipFree(kv.second);
  if (s->part) (void)hipFree(s->part);
  if (s->cnt) (void)hipFree(s->cnt);
  if (s->bar) (void)hipFree(s->bar);
  if (s->err) (void)hipFree(s->err);
  if (s->am_ws) (void)hipFree(s->am_ws);
}

template <class T>
T* upload(const std::vector<T>& v) {
  T* dev = nullptr;
  if (hipMalloc(reinterpret_cast<void**>(&dev), v.size() * sizeof(T)) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (hipMemcpy(dev, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(dev);
    return nullptr;
  }
  return dev;
}

}  // namespace

extern "C" {

int qgemm_seq_create(qgemm_seq_t* out, const qgemm_t* handles, int count, uint32_t flags) {
  if (!out || !handles || count < 1 ||
      (flags & ~(uint32_t)(QGEMM_SEQ_PERSISTENT | QGEMM_SEQ_SUB_BLOCK_SUMS | QGEMM_SEQ_GATED_INPUTS)))
    return QGEMM_EINVAL;
  *out = nullptr;
  int max_R = QGEMM_MAX_R;
  for (int i = 0; i < count; ++i) {
    if (!valid_handle(handles[i])) return QGEMM_EINVAL;
    max_R = std::min(max_R, handles[i]->max_R);
  }
  qgemm_seq* s = new (std::nothrow) qgemm_seq{};
  if (!s) return QGEMM_ENOMEM;
  s->magic = SEQ_MAGIC;
  s->flags = flags;
  s->hs.assign(handles, handles + count);
  if (hipStreamCreateWithFlags(&s->cap, hipStreamNonBlocking) != hipSuccess) {
    s->cap = nullptr;
    delete s;
    return QGEMM_EHIP;
  }
  if (device_cus(&s->cus) != QGEMM_OK) {
    seq_free(s);
    delete s;
    return QGEMM_EHIP;
  }
  s->gated = gated_gemms(s);
  size_t part = 0, cnt = 0;
  if (flags & QGEMM_SEQ_PERSISTENT) {
    // one workgroup per compute unit, all resident
    if (pass_occupancy() < 1) {
      seq_free(s);
      delete s;
      return QGEMM_EPATH;
    }
    bool any = false;
    for (int R = 1; R <= std::min(max_R, PASS_MAX_R); ++R) {
      size_t pr, cn;
      if (!pass_sizes(s, R, &pr, &cn)) continue;
      any = true;
      part = std::max(part, pr);
      cnt = std::max(cnt, cn);
    }
    if (!any) {
      seq_free(s);
      delete s;
      return QGEMM_EPATH;
    }
  }
  part = std::max<size_t>(part, 256);
  cnt = std::max<size_t>(cnt, 256);
  s->part_bytes = part;
  s->cnt_bytes = cnt;
  const size_t bar_bytes = (size_t)PASS_BAR_WORDS * 4;
  s->max_R = max_R;
  const size_t am_bytes = argmax_ws_bytes(max_R, s->hs.back()->N);
  bool ok = hipMalloc(&s->am_ws, am_bytes) == hipSuccess && hipMemset(s->am_ws, 0, am_bytes) == hipSuccess &&
            hipMalloc(reinterpret_cast<void**>(&s->part), part) == hipSuccess &&
            hipMalloc(reinterpret_cast<void**>(&s->cnt), cnt) == hipSuccess &&
            hipMalloc(reinterpret_cast<void**>(&s->bar), bar_bytes) == hipSuccess &&
            hipMalloc(reinterpret_cast<void**>(&s->err), 4) == hipSuccess &&
            hipMemset(s->cnt, 0, cnt) == hipSuccess && hipMemset(s->bar, 0, bar_bytes) == hipSuccess &&
            hipMemset(s->err, 0, 4) == hipSuccess && hipDeviceSynchronize() == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    seq_free(s);
    delete s;
    return QGEMM_ENOMEM;
  }
  *out = s;
  return QGEMM_OK;
}

}  // extern "C"

namespace {

// the whole sequence, then (argmax_idx) the last output's row argmax and
// (tokens) the greedy verification of D drafts per agent, in one epilogue kernel
int seq_run_impl(qgemm_seq_t s, const void* const* xs, float* const* ys, int R, int32_t* argmax_idx,
                 const int32_t* drafts, int D, int32_t* tokens, int32_t* n_new, void* stream) {
  if (!s || s->magic != SEQ_MAGIC || !xs || !ys) return QGEMM_EINVAL;
  if (R < 0) return QGEMM_ERANGE_R;
  for (size_t i = 0; i < s->hs.size(); ++i) {
    if (R > s->hs[i]->max_R) return QGEMM_ERANGE_R;
    if (R > 0 && (!xs[i] || !ys[i])) return QGEMM_EINVAL;
    if (R > 0 && (!aligned16(xs[i]) || !aligned16(ys[i]))) return QGEMM_EALIGN;
  }
  if (R == 0) return QGEMM_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  SeqKey key{R, {}};
  for (size_t i = 0; i < s->hs.size(); ++i) {
    key.ptrs.push_back(reinterpret_cast<uintptr_t>(xs[i]));
    key.ptrs.push_back(reinterpret_cast<uintptr_t>(ys[i]));
  }
  if (!(s->flags & QGEMM_SEQ_PERSISTENT)) {
    // one launch per GEMM, in order, captured once into a graph and replayed
    key.ptrs.push_back(reinterpret_cast<uintptr_t>(argmax_idx));
    key.ptrs.push_back(reinterpret_cast<uintptr_t>(drafts));
    key.ptrs.push_back(reinterpret_cast<uintptr_t>(tokens));
    key.ptrs.push_back(reinterpret_cast<uintptr_t>(n_new));
    key.ptrs.push_back((uintptr_t)D);
    auto g = s->graphs.find(key);
    if (g == s->graphs.end()) {
      if (s->graphs.size() >= SEQ_CACHE_MAX) seq_drop_graphs(s);
      if (hipStreamBeginCapture(s->cap, hipStreamCaptureModeThreadLocal) != hipSuccess) return QGEMM_EHIP;
      int rc = QGEMM_OK;
      for (size_t i = 0; i < s->hs.size() && rc == QGEMM_OK; ++i)
        rc = run_impl(s->hs[i], xs[i], ys[i], R, QGEMM_PATH_AUTO, s->cap);
      if (rc == QGEMM_OK && argmax_idx &&
          launch_argmax_split(ys[s->hs.size() - 1], R, s->hs.back()->N, argmax_idx, s->am_ws, drafts, D, tokens,
                              n_new, s->cap) != hipSuccess)
        rc = QGEMM_EHIP;
      hipGraph_t graph = nullptr;
      const hipError_t e = hipStreamEndCapture(s->cap, &graph);
      if (rc != QGEMM_OK || e != hipSuccess || !graph) {
        if (graph) (void)hipGraphDestroy(graph);
        return rc != QGEMM_OK ? rc : QGEMM_EHIP;
      }
      hipGraphExec_t exec = nullptr;
      const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
      (void)hipGraphDestroy(graph);
      if (ei != hipSuccess) return QGEMM_EHIP;
      g = s->graphs.emplace(key, exec).first;
    }
    return hipGraphLaunch(g->second, st) == hipSuccess ? QGEMM_OK : QGEMM_EHIP;
  }
  // one persistent launch over all GEMMs (pass.hip)
  size_t part, cnt;
  if (!pass_sizes(s, R, &part, &cnt) || part > s->part_bytes || cnt > s->cnt_bytes) return QGEMM_EPATH;
  std::vector<int64_t> mask_off;
  const std::vector<uint64_t> masks = gated_masks(s, R, &mask_off);
  auto mt = s->masks.find(R);
  if (mt == s->masks.end()) {
    uint64_t* dev = upload(masks.empty() ? std::vector<uint64_t>(4, 0) : masks);
    if (!dev) return QGEMM_ENOMEM;
    mt = s->masks.emplace(R, dev).first;
  }
  auto it = s->descs.find(key);
  if (it == s->descs.end()) {
    if (s->descs.size() >= SEQ_CACHE_MAX) seq_drop_descs(s);
    PassGemm* dev = upload(pass_descs(s, R, xs, ys, mt->second, mask_off));
    if (!dev) return QGEMM_ENOMEM;
    it = s->descs.emplace(key, dev).first;
  }
  auto wt = s->waves.find(R);
  if (wt == s->waves.end()) {
    PassWave* dev = upload(pass_waves(pass_descs(s, R, xs, ys, mt->second, mask_off), s->cus));
    if (!dev) return QGEMM_ENOMEM;
    wt = s->waves.emplace(R, dev).first;
  }
  PassArgs a{};
  a.gemms = it->second;
  a.waves = wt->second;
  a.G = (int32_t)s->hs.size();
  a.R = R;
  a.P = s->cus;
  a.part_bytes = (uint32_t)s->part_bytes;
  a.part = s->part;
  a.cnt = s->cnt;
  a.bar = s->bar;
  a.err = s->err;
  a.cnt_half = (uint32_t)(s->cnt_bytes / 8);
  if (launch_pass(a, (s->flags & QGEMM_SEQ_SUB_BLOCK_SUMS) != 0, st) != hipSuccess) return QGEMM_EHIP;
  if (argmax_idx) {
    const qgemm_handle* last = s->hs.back();
    if (launch_argmax_split(ys[s->hs.size() - 1], R, last->N, argmax_idx, s->am_ws, drafts, D, tokens, n_new, st) !=
        hipSuccess)
      return QGEMM_EHIP;
  }
  return QGEMM_OK;
}

}  // namespace

extern "C" {

int qgemm_seq_run(qgemm_seq_t s, const void* const* xs, float* const* ys, int R, int32_t* argmax_idx,
                  void* stream) {
  return seq_run_impl(s, xs, ys, R, argmax_idx, nullptr, 0, nullptr, nullptr, stream);
}

int qgemm_seq_run_verify(qgemm_seq_t s, const void* const* xs, float* const* ys, int R, int32_t* argmax_idx,
                         const int32_t* drafts, int drafts_per_agent, int32_t* tokens, int32_t* n_new,
                         void* stream) {
  if (!argmax_idx || !verify_args_ok(R, drafts, drafts_per_agent, tokens, n_new)) return QGEMM_EINVAL;
  return seq_run_impl(s, xs, ys, R, argmax_idx, drafts, drafts_per_agent, tokens, n_new, stream);
}

int qgemm_seq_errors(qgemm_seq_t s, uint32_t* timeouts) {
  if (!s || s->magic != SEQ_MAGIC || !timeouts) return QGEMM_EINVAL;
  uint32_t v = 0;
  if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(&v, s->err, 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemset(s->err, 0, 4) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
    return QGEMM_EHIP;
  *timeouts = v;
  return QGEMM_OK;
}

int qgemm_seq_destroy(qgemm_seq_t s) {
  if (!s) return QGEMM_OK;
  if (s->magic != SEQ_MAGIC) return QGEMM_EINVAL;
  (void)hipDeviceSynchronize();
  seq_free(s);
  s->magic = 0;
  delete s;
  return QGEMM_OK;
}

}  // extern "C"
