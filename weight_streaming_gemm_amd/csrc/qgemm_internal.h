// qgemm_internal.h — kernel arguments and launch wrappers shared by the kernel
// and API translation units of the library (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "prefill_plan.h"

namespace qg {

// One GEMM of a launch: y[R x N] = x[R x K] . W^T over packed weights.
struct GemmDesc {
  const uint8_t* packed;   // quant region (quant_bytes), then the header region (hdr_bytes)
  const uint16_t* x;       // bf16 activations, R x K row-major
  float* y;                // fp32 outputs, R x N row-major
  uint32_t quant_bytes;    // < 2^31
  uint32_t hdr_bytes;
  int32_t N, NS, KB;       // outputs, 16-output sub-tiles, 256-weight blocks
  int32_t nwn;             // waves of a workgroup side by side along N (the other
                           // NW / nwn split each range along K)
  int32_t T;               // output tiles of nwn * NT sub-tiles
  int32_t I;               // T * KB (tile, block) steps
  int32_t V;               // contiguous step ranges (P <= V <= I); workgroup p takes
                           // ranges p, p + P, p + 2P, ...
  int32_t aligned;         // 0: V equal ranges of steps; 1: V ranges of whole tiles
                           // (tiles [floor(v T / V), floor((v + 1) T / V))), so that
                           // no tile is shared between ranges
  // K in S chunks (S > 1 when a tile row of activations does not fit in LDS):
  // tile t above is then chunk t / treal of output tile t mod treal, KB above is
  // the chunk's blocks and kbr the row's; each chunk of a tile leaves a partial
  // result, and the last chunk to arrive adds the S of them in chunk order.
  int32_t S, kbr, treal;
  int32_t pad_;
};

// A launch of the streaming kernel (one GEMM).
struct StreamArgs {
  GemmDesc d0;             // the GEMM
  float* part;             // 2 V partial-tile slots of nwn * NT * RT KiB
  uint32_t* cnt;           // per-tile arrival counters, zero between launches
  int32_t R, P;
  int32_t RT, NT, NW;
  int32_t msum;            // 1: min term from sub-block sums staged with the
                           // activations (one product per step); 0: from the
                           // activations themselves (eight products per step)
  int32_t valu;            // 1: vector-unit variant (R <= 4, msum = 1, one GEMM)
};
constexpr int MAX_ROWS = 64;        // rows of a run (QGEMM_MAX_R)
constexpr int VALU_MAX_R = 4;       // rows the vector-unit kernel serves
constexpr int VALU_AUTO_MAX_R = 0;  // rows for which the automatic choice takes it

// Kernel variants: (row tiles RT, sub-tiles per tile NT, waves per workgroup NW).
// A workgroup (one per CU) holds in LDS the partial tiles of its waves (two per
// wave) and the activations of the blocks its current range touches (and their
// sub-block sums when they are used), in what is left of 160 KiB.
constexpr int LDS_BYTES = 160 * 1024;
constexpr int LDS_RESERVED = 1024;              // flags
inline constexpr int piece_bytes(int RT, int NT, int NW) { return NW * 2 * NT * RT * 1024; }
inline constexpr int x_area_bytes(int RT, int NT, int NW) { return LDS_BYTES - LDS_RESERVED - piece_bytes(RT, NT, NW); }
inline int x_slot_bytes(int R, bool msum) { return 8 * (64 * R + 16) + (msum ? 32 * R : 0); }
inline int x_slot_capacity(int R, int RT, int NT, int NW, bool msum) {
  return x_area_bytes(RT, NT, NW) / x_slot_bytes(R, msum);
}
inline int waves_for(int RT) { (void)RT; return 8; }   // two waves per SIMD at every row count
inline int subtiles_for(int RT) { (void)RT; return 1; }
inline size_t partial_slot_bytes(int RT, int NT, int nwn) { return (size_t)nwn * NT * RT * 1024; }

hipError_t launch_pack(const uint8_t* canon, uint8_t* packed, int64_t N, int64_t K, hipStream_t st);
hipError_t launch_stream(const StreamArgs& a, hipStream_t st);
hipError_t launch_read_probe(const void* buf, uint64_t bytes, void* sink, int cus, hipStream_t st);
bool stream_variant_exists(int RT, int NT, int NW);
int stream_occupancy(int RT, int NT, int NW);   // resident workgroups per CU (0 if no such variant)
// rows tiled as well as outputs (prefill.hip; plan and image layout in prefill_plan.h):
// x [R x K] bf16, y [R x N] fp32, any R
hipError_t launch_prefill(const uint8_t* packed, int64_t N, int64_t K, const void* x, float* y, int R,
                          const PrefillPlan& p, void* ws, hipStream_t st);
hipError_t launch_dequant(const uint8_t* packed, float* w, int64_t N, int64_t K, hipStream_t st);
hipError_t launch_argmax(const float* y, int R, int64_t N, int32_t* idx, hipStream_t st);
// Row argmax over column chunks with a workspace of argmax_ws_bytes(R, N) bytes
// (chunk partials, then R + 1 arrival counters that start and end at zero);
// with tokens != null the kernel also runs the greedy draft verification.
inline int argmax_chunks(int64_t N) {
  const int64_t c = (N + 8191) / 8192;
  return (int)(c < 1 ? 1 : (c > 1024 ? 1024 : c));
}
inline size_t argmax_ws_bytes(int R, int64_t N) {
  return (((size_t)R * argmax_chunks(N) * 8 + (size_t)(R + 1) * 4) + 15) / 16 * 16;
}
hipError_t launch_argmax_split(const float* y, int R, int64_t N, int32_t* idx, void* ws, const int32_t* drafts,
                               int D, int32_t* tokens, int32_t* n_new, hipStream_t st);
hipError_t launch_verify(const int32_t* idx, int R, const int32_t* drafts, int D, int32_t* tokens, int32_t* n_new,
                         hipStream_t st);

// ---- the persistent pass kernel (pass.hip, schedule in pass_sched.h) ----------
// One GEMM of the sequence, as the kernel reads it from a device table.
struct PassGemm {
  const uint8_t* qbase;    // quant region (qbytes), header region (hbytes) of the packed weights
  const uint8_t* hbase;
  uint32_t qbytes, hbytes;
  const uint16_t* x;       // bf16 activations, R x K row-major
  float* y;                // fp32 outputs, R x N row-major
  int32_t N, NS, KB;       // outputs, 16-output sub-tiles, 256-weight blocks
  int32_t S, kbc;          // K in S chunks of kbc blocks
  int32_t rot;             // rotation of the deal of units to workgroups
  // gated input (the previous GEMM is a fused gate|up of 2 K outputs feeding this
  // one through an element-wise gate): per chunk c, PASS_MASK_WORDS words: a
  // 256-bit mask of the workgroups whose units of the previous GEMM hold the
  // outputs the chunk reads, then the value the chunk's counter reaches once they
  // have all finished (counts add up over the launch's gated GEMMs); a workgroup
  // of chunk c waits only for that.  NULL: wait for every workgroup.
  const uint64_t* masks;
};
// A compute wave's share of one GEMM (pass_sched.h), precomputed on the host:
// `count` steps starting at packed step `step0` (sub-tile * KB + block), at
// block `jj0` of the chunk; `next` = the first later GEMM where the wave has
// steps (G if none).
struct PassWave {
  int32_t count, step0, jj0, next;   // steps, first packed step and block, next GEMM with steps
  int32_t xblk;                      // activation blocks the workgroup stages (0: no units)
};
struct PassArgs {
  const PassGemm* gemms;   // device table of G GEMMs
  const PassWave* waves;   // device table [G][P][PASS_NC]
  int32_t G, R, P;         // GEMMs, rows (1..PASS_MAX_R), workgroups (all resident)
  uint32_t part_bytes;     // bytes of `part` (two halves: GEMMs of even and odd index)
  float* part;             // chunk partial tiles: chunk c, sub-tile ns at (c NS + ns) KiB of a half
  uint32_t* cnt;           // per-sub-tile chunk arrival counters (two halves, as `part`), zero
                           // between uses
  uint32_t* bar;           // PASS_BAR_WORDS barrier counters, zero between launches
  uint32_t* err;           // set to 1 when a device-wide wait gave up
  uint32_t cnt_half;       // words of one half of `cnt`
  uint32_t pad_;
};
constexpr int PASS_MAX_RT = 3;                   // row tiles of 16 rows
constexpr int PASS_MAX_R = 16 * PASS_MAX_RT;
inline constexpr int pass_row_tiles(int R) { return (R + 15) / 16; }
constexpr int PASS_NC = 8;                       // compute waves per workgroup
constexpr int PASS_NH = 4;                       // helper waves per workgroup
constexpr int PASS_THREADS = (PASS_NC + PASS_NH) * 64;
constexpr int PASS_PIECES = 2;                   // LDS partial tiles per compute wave
constexpr int PASS_RING = 8;                     // weight steps in flight per compute wave (1-2 row tiles)
inline constexpr int pass_ring(int RT) { return RT <= 2 ? PASS_RING : 7; }   // registers left at 3 row tiles
constexpr int PASS_MAX_CHUNKS = 32;
// at one row tile the last chunk to arrive adds a sub-tile's partial tiles in one
// round of 16 loads: at most 16 chunks there
inline constexpr int pass_max_chunks(int RT) { return RT == 1 ? 16 : PASS_MAX_CHUNKS; }
// barrier words: bar[0] global counter, bar[16] exit counter, bar[32 + 32 k] group k's
// counter, bar[512 + 32 k] group k's release word (k < 8)
constexpr int PASS_RELEASE_WORD = 512;
constexpr int PASS_DEP_WORD = 1024;              // bar[1024 + 256 c]: gated-input counter of chunk c
constexpr int PASS_DEP_STRIDE = 256;             // (one KiB apart)
constexpr int PASS_BAR_WORDS = PASS_DEP_WORD + PASS_MAX_CHUNKS * PASS_DEP_STRIDE;
constexpr int PASS_MAX_GATED_P = 256;            // workgroups a gated wait's bitmask covers
constexpr int PASS_MASK_WORDS = 8;               // per gated chunk: 4 words of bitmask, the counter's target
// piece slots per compute wave at RT row tiles (one slot from two row tiles on,
// so that the activations keep the LDS of one row tile's two slots), and the LDS
// bytes for activations: what the pieces (RT KiB each) and a few words leave of 160 KiB
inline constexpr int pass_pieces(int RT) { return RT == 1 ? PASS_PIECES : 1; }
inline constexpr int pass_x_area(int RT) { return 160 * 1024 - PASS_NC * pass_pieces(RT) * RT * 1024 - 256; }
hipError_t launch_pass(const PassArgs& a, bool msum, hipStream_t st);
int pass_occupancy();                            // resident workgroups per CU (0: none)

// The allocation-free entry point's fixed device scratch (qgemm_run_static):
// its bytes, its address on the current device, and a kernel that zeroes words.
constexpr size_t STATIC_SCRATCH_BYTES = size_t(16) << 20;
hipError_t static_scratch_address(void** out);
hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t st);

}  // namespace qg
