// Internal declarations shared by the host runtime and the gfx950 kernels of
// the walk-resident serial draft head ("Weights That Stay", arXiv 2611.00506).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wts {

constexpr int kR = 256;           // latent rank the kernels are built for
constexpr int kTileRows = 16;     // vocabulary rows per W tile (one MFMA N block)
constexpr int kWaves = 8;         // waves per workgroup of the persistent kernel (at most)
constexpr int kThreads = kWaves * 64;
constexpr int kMaxB = 16;
constexpr int kMaxSteps = 64;
// Waves per workgroup of the persistent kernel.  bf16 Markov walks use 4
// waves (one per SIMD): each wave then has the whole 512-entry register file
// of its SIMD lane (VGPRs + AGPRs) and keeps 8 bf16 tiles (64 KiB per wave)
// resident; everything else uses 8 waves.
constexpr int waves_for(int head, int wtype) { return (head == 0 && wtype == 1) ? 4 : 8; }
// 16-row W tiles a wave of the persistent kernel holds in registers.  Larger
// batches need more registers for latents and keys, so they keep fewer tiles
// in registers and more in LDS.  At two to eight int8 Markov rows the fifth
// register tile fits only in greedy walks without the log normaliser (T=1
// keys and noise, or the running log-sum-exp pairs, would spill); the same
// holds for one extra bf16 tile at four, eight and sixteen rows.
// The recurrent head also keeps its matrix-vector partial results across the
// step, so it holds fewer.
constexpr int reg_tiles_max(int head, int wtype, int BB, int temp, bool ls) {
  return wtype == 0 ? (head == 0 ? (BB == 1 ? 5 : BB <= 8 ? (temp == 0 && !ls ? 5 : 4) : 2)
                                 : (BB == 1 ? 5 : BB == 2 ? 4 : BB == 4 ? 3 : BB == 8 ? 2 : 1))
                    : waves_for(head, wtype) == 4 ? (BB == 1 ? 9 : BB == 2 ? 8 : BB <= 4 ? (temp == 0 && !ls ? 8 : 7) : BB == 8 ? (temp == 0 && !ls ? 7 : 6) : (temp == 0 && !ls ? 7 : 5)) : 1;
}
// Register tiles per wave of the whole-shard-on-chip variant (bf16 Markov
// walks of up to four batch rows): without streaming buffers a wave can hold
// more W in registers, and LDS tiles are handed out per wave as needed, so
// the bf16 shard of a 248k vocabulary (61 tiles per CU) stays on chip.  0: no
// such variant.  kFullLdsMax: LDS tiles a wave of that variant may own.
constexpr int reg_tiles_full(int head, int wtype, int BB) { return (head == 0 && wtype == 1 && BB <= 4) ? 11 : 0; }
constexpr int kFullLdsMax = 6;
constexpr int kChunksI8 = 4;      // 16-byte lane chunks per int8 tile (64 k each)
constexpr int kChunksBF = 8;      // 16-byte lane chunks per bf16 tile (32 k each)
constexpr int kTileBytesI8 = kTileRows * kR;       // 4 KiB
constexpr int kTileBytesBF = kTileRows * kR * 2;   // 8 KiB
// LDS of the persistent kernel: scratch for reductions and the latent, then
// W tiles.  Asking for more than half of the 160 KiB also pins one workgroup
// per compute unit.
constexpr int kLdsMax = 163840;

constexpr int kHeadMarkov = 0;
constexpr int kHeadRecurrent = 1;

// Walks of one batch row stage the embedding rows of the exchange's
// candidates (the group maxima) in LDS while the exchange runs: int8 Markov
// walks (E_q rows) and recurrent walks (fp32 E rows).
constexpr bool stage_candidates(int head, int wtype, int BB) {
  return BB == 1 && (head == kHeadRecurrent || wtype == 0);
}
// LDS bytes in front of the LDS-resident W tiles.
constexpr int lds_scratch_bytes(int head, int wtype, int BB) {
  return head == kHeadRecurrent ? 32768 + kR * kR * 2 : stage_candidates(head, wtype, BB) ? 21504 : 5120;
}
// LDS offset of the log-sum-exp pairs: per wave and batch row (float2
// [kWaves][kMaxB], 1 KiB), then the exchange wave's raw pairs (float2
// [result entries][64], at most 2 KiB; 1 KiB at B=1), in a part of the
// scratch that nothing else of that kernel uses.
constexpr int lse_lds_offset(int head, int wtype, int BB) {
  return head == kHeadRecurrent ? (BB == 1 ? 29696 : 27136) : stage_candidates(head, wtype, BB) ? 18688 : 2048;
}

constexpr int kMaxGrid = 256;   // workgroups of the persistent kernel at most
constexpr int kGroups = 16;     // first level of the cross-workgroup selection
constexpr int kCopies = 8;      // copies of the second-level lines (one per XCD)
constexpr int kSub = 16;        // step-wise path: sub-slots per (step, batch row)

// Device control block of one context.  Every array has a leading walk
// parity: a walk reads `epoch` when it starts and uses parity epoch & 1, its
// first launch clears the arrays of the other parity for the next walk, and
// its last act advances `epoch` (the persistent walk: workgroup 0 after its
// last exchange; the step-wise walk: its finishing launch).  No host-side
// state or reset is needed between walks, so a walk captured once in a graph
// can be replayed.
struct Ctrl {
  // persistent walk, two-level all-gather of tagged keys (step parity second)
  unsigned long long l1[2][2][kMaxGrid][kMaxB];   // one line per workgroup
  unsigned long long l2[2][2][kCopies][kGroups][kMaxB];  // one line per group and copy
  // step-wise walk: device-scope max per (step, batch row, sub-slot)
  unsigned long long ss[2][kMaxSteps][kMaxB][kSub];
  unsigned int err;                               // latched wts_status
  unsigned int epoch;                             // walks completed (their parity alternates)
  unsigned int pad[62];
};

struct WalkArgs {
  // from the context
  const int4* Wp;          // tile-major W: [tiles][chunks][64 lanes] x 16 B
  const float* sw;         // [tiles * 16] per-row scale (int8), 0 on pad rows
  const int8_t* Eq;        // [V][512]: hi[256] | lo[256] of each E row (int8)
  const float* Es;         // [V] s_hi of each E row (int8 Markov)
  const uint16_t* Eb;      // [V][256] bf16 E rows (bf16 Markov)
  const float* E;          // [V][256] fp32 (recurrent)
  const uint16_t* A;       // [256][256] bf16 (recurrent)
  const float* c;          // [256] (recurrent)
  Ctrl* ctrl;
  int V;
  int tiles;
  int head;
  int reg_tiles;           // per wave, in registers
  int lds_tiles;           // per wave, in LDS
  int lds_extra;           // waves 0 .. lds_extra - 1 hold one LDS tile more (walks that stream)
  int noise_off;           // T=1 persistent Markov walks: LDS offset of the noise rows, else 0
  int noise_stride;        // floats per batch row in that buffer (>= rows of a workgroup)
  // of this walk
  int B;
  int gamma;
  int step_offset;
  int temperature;
  unsigned seed_lo;
  unsigned seed_hi;
  int step;                // step-wise launches: the step this launch runs
  const uint16_t* base;
  unsigned base_bytes;     // 2 B gamma V: the base logits' bytes (below 2^32)
  const int* x0;
  const float* h0;
  int* tokens;
  uint16_t* logits;
  float* state;
  long long* trace;        // [gamma][grid][4] phase stamps or null
  long long timeout_ticks; // watchdog, in s_memrealtime ticks (100 MHz)
  int fixed_latent;        // fixed-latent probe: the latent of step 0 at every step
  int full;                // whole shard on chip (reg_tiles_full variant); lds tiles allotted per wave
  float* lse;              // [B][gamma] log normaliser per step, or null
  float* lse_part;         // [B][gamma][grid] (max, sum) pairs of the workgroups (scratch)
  int xcd_l1;              // 1: first exchange level inside one XCD's L2; 0: device scope
  int stress;              // pseudo-random delay of every workgroup before each exchange
  unsigned long long* winners;  // [gamma][B][grid] winning key each workgroup observed, or null
};

// Launchers (wts_kernels.hip).  Each returns the HIP error of its launch.
hipError_t launch_repack_i8(const int8_t* W, const float* w_scale, int V, int tiles,
                            int4* Wp, float* sw, hipStream_t s);
hipError_t launch_repack_bf16(const uint16_t* W, int V, int tiles, int4* Wp, hipStream_t s);
hipError_t launch_quant_rows(const float* E, int V, int8_t* Eq, float* Es, hipStream_t s);
hipError_t launch_bf16_rows(const float* E, int V, uint16_t* Eb, hipStream_t s);
hipError_t launch_walk(int wtype, int BB, const WalkArgs& a, int grid, int lds_bytes,
                       bool cooperative, hipStream_t s);
hipError_t launch_step(int wtype, int BB, const WalkArgs& a, int grid, hipStream_t s);
hipError_t launch_finish(const WalkArgs& a, hipStream_t s);
hipError_t launch_lse(const WalkArgs& a, int grid, hipStream_t s);
hipError_t launch_check_log_ratio(unsigned long long* mismatches, hipStream_t s);
hipError_t prepare_kernels(int lds_bytes);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_xcc_ids(unsigned* out, int grid, hipStream_t s);
// roofline microbenchmarks (wts_roofline.hip drives them)
hipError_t launch_rf_lds(int grid, int rounds, unsigned* out, hipStream_t s);
hipError_t launch_rf_mfma(int wtype, int grid, int rounds, unsigned* out, long long* clk, hipStream_t s);
hipError_t launch_rf_stream(const void* p, long long n16, int passes, int grid, unsigned* out, hipStream_t s);
hipError_t launch_rf_exchange(int variant, int grid, int rounds, Ctrl* ctrl, unsigned long long* flat, unsigned* cnt,
                              long long timeout, long long* clk, unsigned* wrong, hipStream_t s);
hipError_t launch_rf_pingpong(int grid, int peer, int xcd, int rounds, unsigned long long* flag, long long timeout,
                              long long* clk, hipStream_t s);
hipError_t launch_rf_valu(int mode, int waves, int n, float* out, long long* clk, hipStream_t s);

}  // namespace wts
