// gfx950 kernels of the walk-resident serial draft head.
//
// Method: "Weights That Stay: On-Chip Megakernels for Serial Heads in
// Speculative Decoding" (arXiv 2611.00506).  One persistent launch runs the
// whole gamma-step walk (Fig. 1, Fig. 4): each workgroup keeps its shard of
// the vocabulary projection W on chip, projects the step's latent through it,
// selects a local winner, all workgroups agree on the common winner (Fig. 8),
// and the state advances in the kernel.  int8 W uses the two-int8-vector
// latent of Fig. 7; bf16 W uses the latent rounded to bf16.
//
// MI355X mapping (not the pages' H100/B200 design):
//  * one workgroup per CU, of 8 waves (4 for bf16 Markov walks, which need a
//    whole SIMD's register file per wave); a wave owns every NW-th 16-row tile
//    of its workgroup's contiguous tile range;
//  * a tile is one MFMA N block: the latent rows are the A operand (16 x K),
//    the 16 vocabulary rows of the tile the B operand (K x 16), so the
//    projection of a step is a chain of v_mfma_i32_16x16x64_i8 (int8 W) or
//    v_mfma_f32_16x16x32_bf16 (bf16 W) per tile;
//  * when the batch leaves A rows unused, the A operand repeats the latent
//    rows in every slot of RPS rows, S tiles run against it with their own
//    accumulators, and the lanes of result slot s take tile s, so all 64 lanes
//    of the result carry useful logits;
//  * W tiles live in registers, then LDS, and the remainder streams from HBM
//    each step with one or two tiles of prefetch; a whole-shard variant (bf16,
//    up to four batch rows) drops the streaming buffers to hold more tiles in
//    registers;
//  * the cross-workgroup selection is a two-level all-gather of step-tagged
//    64-bit keys (one line per workgroup, a group leader per 16 workgroups,
//    one line per group and XCD), polled by one wave per workgroup with a
//    wall-clock watchdog.  The first level stays inside one XCD's L2.  Fig. 8
//    has each worker atomically update one maximum and an arrival count; on
//    MI355X that serialises 2 x 256 device-scope atomics per step (measured
//    about 10 us per round), and the all-gather needs none.
//
// Bit-exactness with the oracle needs: no contraction of a*b+c (built with
// -ffp-contract=off), IEEE division (default), rintf half-even.

#include "wts_internal.h"

namespace wts {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// ----------------------------------------------------------------------------
// scalar helpers
// ----------------------------------------------------------------------------

// bf16 = upper half of binary32, rounded to nearest even (Fig. 7: the
// logit is rounded to bf16 a single time).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t b = __float_as_uint(x);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return b >> 16;
}
__device__ __forceinline__ float bf16_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Selection key (Fig. 8: each worker's local winner as one key): bits 49..18 order the
// binary32 scores (-0 folded into +0), bits 17..0 hold 0x3FFFF - v so the
// lowest index wins among equal scores (V < 2^18).  0 is below every key.
// Bits 63..57 are left free for the step tag of the cross-workgroup exchange.
constexpr unsigned long long kKeyMask = (1ull << 50) - 1;
constexpr int kTagShift = 57;
__device__ __forceinline__ unsigned long long sel_key(float s, int v) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)o << 18) | (unsigned long long)(0x3FFFFu - (uint32_t)v);
}
__device__ __forceinline__ int key_token(unsigned long long k) { return (int)(0x3FFFFu - (uint32_t)(k & 0x3FFFFu)); }
__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}

// Portable elementary functions, one binary32 operation at a time.
// log: x = m 2^e, m in [sqrt(1/2), sqrt(2)); log m = 2 atanh(s), s = (m-1)/(m+1),
// series through s^9; ln 2 split in a high part exact for |e| <= 256 and a
// low part (Cody-Waite).
constexpr float kLn2Hi = 0.693145751953125f;
constexpr float kLn2Lo = (float)(0.69314718055994530942 - 0.693145751953125);
constexpr float kInvLn2 = (float)(1.0 / 0.69314718055994530942);
constexpr float kLogC9 = (float)(1.0 / 9.0);
constexpr float kLogC7 = (float)(1.0 / 7.0);
constexpr float kLogC5 = (float)(1.0 / 5.0);
constexpr float kLogC3 = (float)(1.0 / 3.0);

// s = f / (2 + f) for the reduced argument of log_p (f = m - 1 with m in
// [sqrt(1/2), sqrt(2))): a reciprocal estimate of the denominator, the
// quotient, its exact residual (fused multiply-add) and one correction.  For
// every f that log_p can produce this equals the correctly rounded binary32
// quotient (all 2^23 reduced mantissas are compared with the IEEE division
// on the device by check_log_ratio_kernel); it takes 4 instructions against
// about 10 for the general division.
__device__ __forceinline__ float log_ratio(float f) {
  const float d = 2.0f + f;
  const float r = __builtin_amdgcn_rcpf(d);
  const float q = f * r;
  const float e = __builtin_fmaf(-q, d, f);
  return __builtin_fmaf(e, r, q);
}

__device__ float log_p(float x) {
  const uint32_t bits = __float_as_uint(x);
  int e = (int)((bits >> 23) & 0xFFu) - 126;
  float m = __uint_as_float((bits & 0x007FFFFFu) | 0x3F000000u);
  if (m < 0.70710677f) {
    m = m * 2.0f;
    e = e - 1;
  }
  const float f = m - 1.0f;
  const float s = log_ratio(f);
  const float z = s * s;
  float p = kLogC9 * z;
  p = (p + kLogC7) * z;
  p = (p + kLogC5) * z;
  p = (p + kLogC3) * z;
  const float lm = 2.0f * (s + s * p);
  const float ef = (float)e;
  return ef * kLn2Hi + (ef * kLn2Lo + lm);
}

// e^y for y in [-20, 0]: n = rint(y / ln 2), reduced argument, degree-8
// Taylor polynomial (Horner), exact scaling by 2^n.
__device__ float exp_p(float y) {
  const float n = rintf(y * kInvLn2);
  const float f = (y - n * kLn2Hi) - n * kLn2Lo;
  float p = (float)(1.0 / 40320.0);
  p = p * f + (float)(1.0 / 5040.0);
  p = p * f + (float)(1.0 / 720.0);
  p = p * f + (float)(1.0 / 120.0);
  p = p * f + (float)(1.0 / 24.0);
  p = p * f + (float)(1.0 / 6.0);
  p = p * f + 0.5f;
  p = p * f + 1.0f;
  p = p * f + 1.0f;
  const float scale = __uint_as_float((uint32_t)((int)n + 127) << 23);
  return p * scale;
}

// tanh: odd Taylor series below 1/4, (1 - e^{-2a}) / (1 + e^{-2a}) up to 10,
// 1 beyond; sign of x restored.
__device__ float tanh_p(float x) {
  const float a = fabsf(x);
  if (a < 0.25f) {
    const float x2 = x * x;
    float t = (float)(-1382.0 / 155925.0);
    t = t * x2 + (float)(62.0 / 2835.0);
    t = t * x2 + (float)(-17.0 / 315.0);
    t = t * x2 + (float)(2.0 / 15.0);
    t = t * x2 + (float)(-1.0 / 3.0);
    return x + x * (x2 * t);
  }
  float r = 1.0f;
  if (a < 10.0f) {
    const float q = exp_p(-2.0f * a);
    r = (1.0f - q) / (1.0f + q);
  }
  return x < 0.0f ? -r : r;
}

// Both halves of a 32x32->64 product from one instruction (v_mad_u64_u32)
// rather than separate high and low multiplies.
__device__ __forceinline__ void mul_wide(uint32_t m, uint32_t x, uint32_t& hi, uint32_t& lo) {
  const uint64_t p = (uint64_t)m * (uint64_t)x;
  hi = (uint32_t)(p >> 32);
  lo = (uint32_t)p;
}

// Philox4x32-10 (Salmon et al., SC'11): 10 rounds of two 32x32->64 products,
// Weyl key schedule between rounds.  Noise for (b, step, v): counter
// (v >> 2, step, b, 0), key (seed_lo, seed_hi), output word v & 3.
__device__ float gumbel(uint32_t k0, uint32_t k1, int b, int step, int v) {
  uint32_t c0 = (uint32_t)v >> 2, c1 = (uint32_t)step, c2 = (uint32_t)b, c3 = 0u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    uint32_t hi0, lo0, hi1, lo1;
    mul_wide(0xD2511F53u, c0, hi0, lo0);
    mul_wide(0xCD9E8D57u, c2, hi1, lo1);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  const int sel = v & 3;
  const uint32_t w = sel == 0 ? c0 : sel == 1 ? c1 : sel == 2 ? c2 : c3;
  // U = (2 (w >> 9) + 1) 2^-24, exact, in (0, 1)
  const float u = (float)(2u * (w >> 9) + 1u) * 5.9604644775390625e-08f;
  const float y = -log_p(u);
  return -log_p(y);
}

// ----------------------------------------------------------------------------
// create-time kernels
// ----------------------------------------------------------------------------

// W [V][256] int8 -> tile-major [tile][chunk c<4][lane] x 16 B, where lane
// l carries row 16*tile + (l & 15), columns 64c + 16(l >> 4) .. +16 -- the B
// operand of v_mfma_i32_16x16x64_i8 for that chunk.  Pad rows are zero.
__global__ void repack_i8_kernel(const int8_t* __restrict__ W, const float* __restrict__ ws,
                                 int V, int tiles, int4* __restrict__ Wp, float* __restrict__ sw) {
  const long long id = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)tiles * kChunksI8 * 64;
  if (id >= total) return;
  const int lane = (int)(id & 63);
  const int c = (int)((id >> 6) % kChunksI8);
  const int tile = (int)(id / (64 * kChunksI8));
  const int row = tile * kTileRows + (lane & 15);
  int4 v = make_int4(0, 0, 0, 0);
  if (row < V) v = *(const int4*)(W + (size_t)row * kR + c * 64 + (lane >> 4) * 16);
  Wp[id] = v;
  if (c == 0 && lane < 16) sw[tile * kTileRows + lane] = row < V ? ws[row] : 0.0f;
}

// W [V][256] bf16 -> [tile][chunk c<8][lane] x 16 B: row 16*tile + (l & 15),
// columns 32c + 8(l >> 4) .. +8 (B operand of v_mfma_f32_16x16x32_bf16).
__global__ void repack_bf16_kernel(const uint16_t* __restrict__ W, int V, int tiles,
                                   int4* __restrict__ Wp) {
  const long long id = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)tiles * kChunksBF * 64;
  if (id >= total) return;
  const int lane = (int)(id & 63);
  const int c = (int)((id >> 6) % kChunksBF);
  const int tile = (int)(id / (64 * kChunksBF));
  const int row = tile * kTileRows + (lane & 15);
  int4 v = make_int4(0, 0, 0, 0);
  if (row < V) v = *(const int4*)(W + (size_t)row * kR + c * 32 + (lane >> 4) * 8);
  Wp[id] = v;
}

// Wave-wide maximum of a float (all lanes get the result).
// Maximum of a non-negative float over the wave: DPP maxima inside each
// 16-lane row (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror), then the four rows via readlane.  For x >= 0 the bit patterns
// order as the values do.
__device__ __forceinline__ float wave_max_nonneg(float x) {
  uint32_t b = __float_as_uint(x);
#define WTS_QMAX(c) b = max(b, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)b, (c), 0xF, 0xF, false))
  WTS_QMAX(0xB1);
  WTS_QMAX(0x4E);
  WTS_QMAX(0x141);
  WTS_QMAX(0x140);
#undef WTS_QMAX
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)b, 0), r1 = (uint32_t)__builtin_amdgcn_readlane((int)b, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)b, 32), r3 = (uint32_t)__builtin_amdgcn_readlane((int)b, 48);
  return __uint_as_float(max(max(r0, r1), max(r2, r3)));
}

// Two-int8-vector latent of one 256-vector held 4 values per lane (Fig. 7):
// symmetric absmax scale s_hi = amax/127, hi = rint(u 127/amax), residual
// r = u - s_hi hi, lo = rint(r 256 * 127/amax), both clamped to +-127,
// s_lo = s_hi / 256.  Returns s_hi; hi/lo of elements 4*lane..+3 in *hi,*lo.
__device__ __forceinline__ float quant4(const float u[4], uint32_t* hi4, uint32_t* lo4) {
  float amax = fmaxf(fmaxf(fabsf(u[0]), fabsf(u[1])), fmaxf(fabsf(u[2]), fabsf(u[3])));
  amax = wave_max_nonneg(amax);
  uint32_t ph = 0, pl = 0;
  float s_hi = 0.0f;
  if (amax != 0.0f) {
    s_hi = amax / 127.0f;
    const float inv = 127.0f / amax;
    const float inv256 = inv * 256.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float h = rintf(u[i] * inv);
      h = fminf(fmaxf(h, -127.0f), 127.0f);
      const float res = u[i] - s_hi * h;
      float l = rintf(res * inv256);
      l = fminf(fmaxf(l, -127.0f), 127.0f);
      ph |= ((uint32_t)(int)h & 0xFFu) << (8 * i);
      pl |= ((uint32_t)(int)l & 0xFFu) << (8 * i);
    }
  }
  *hi4 = ph;
  *lo4 = pl;
  return s_hi;
}

// E [V][256] fp32 -> Eq [V][512] (hi | lo) and Es [V] (s_hi).  One wave per row.
__global__ void quant_rows_kernel(const float* __restrict__ E, int V, int8_t* __restrict__ Eq,
                                  float* __restrict__ Es) {
  const int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= V) return;  // whole wave leaves together
  const float4 u4 = *(const float4*)(E + (size_t)row * kR + lane * 4);
  const float u[4] = {u4.x, u4.y, u4.z, u4.w};
  uint32_t h, l;
  const float s = quant4(u, &h, &l);
  *(uint32_t*)(Eq + (size_t)row * 512 + lane * 4) = h;
  *(uint32_t*)(Eq + (size_t)row * 512 + 256 + lane * 4) = l;
  if (lane == 0) Es[row] = s;
}

// E [V][256] fp32 -> bf16 rows.
__global__ void bf16_rows_kernel(const float* __restrict__ E, long long n, uint16_t* __restrict__ Eb) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) Eb[i] = (uint16_t)bf16_rne(E[i]);
}

// ----------------------------------------------------------------------------
// the walk
// ----------------------------------------------------------------------------

// Geometry of one (W type, batch bucket).  The A operand carries LPB latent
// rows per batch row (hi and lo for int8, one for bf16).  With RPS latent
// rows per slot, S = 16 / RPS tiles share one A operand, each with its own
// accumulator, and the lanes of result slot s take tile s.
template <int WT, int BB, int HD = 0, bool FL = false, int TP = 0, bool LSP = false>
struct Geo {
  static constexpr int LPB = WT == 0 ? 2 : 1;
  static constexpr int ROWS = LPB * BB;
  static constexpr int NM = ROWS > 16 ? ROWS / 16 : 1;
  static constexpr int RPS = ROWS <= 4 ? 4 : (ROWS <= 8 ? 8 : 16);
  static constexpr int S = 16 / RPS;
  static constexpr int CH = WT == 0 ? kChunksI8 : kChunksBF;
  static constexpr int RT = FL ? reg_tiles_full(HD, WT, BB) : reg_tiles_max(HD, WT, BB, TP, LSP);
  static constexpr int NG = (RT + S - 1) / S;
  static constexpr int NE = 4 / LPB;  // batch entries per lane and M block
};

// LDS map of the persistent and step kernels.
constexpr int kOffRed = 0;                       // u64 [kWaves][kMaxB]
constexpr int kOffX = kOffRed + 8 * kWaves * kMaxB;   // int [kMaxB]
constexpr int kOffShi = kOffX + 4 * kMaxB;        // float [kMaxB]
constexpr int kOffFlag = kOffShi + 4 * kMaxB;     // int
constexpr int kOffDone = kOffFlag + 8;           // int: step + 1 whose exchange finished
constexpr int kOffWin = kOffDone + 8;            // int [kMaxB]: staged row holding the winner
constexpr int kOffLseCnt = 1240;                 // int: waves done with this step's log-sum-exp pairs
constexpr int kOffZero = 1280;                   // 256 zero bytes (A-operand source of other slots)
constexpr int kOffCand = 1536;                   // u64 [kGroups][2]: group maxima seen so far
// Staged candidate rows: hi at 0, lo at kLoOff of each row.  The 64-byte gap
// puts the 16-byte chunks of the two halves that one A-operand read fetches
// together (same k chunk, alternate A rows) in disjoint LDS banks.
constexpr int kOffRows = 2048;                   // [kGroups][kRowBytes]
constexpr int kLoOff = 320;
constexpr int kRowBytes = kLoOff + 256;
constexpr int kOffShs = kOffRows + kGroups * kRowBytes;  // float [kGroups]: their s_hi
static_assert(kLoOff % 64 == 0 && kLoOff >= 256, "lo half past the hi half, on a 64-byte boundary");
static_assert(kOffShs + 4 * kGroups <= lse_lds_offset(kHeadMarkov, 0, 1), "staged rows below the lse pairs");
// Latent rows the recurrent head builds in LDS, 16 bytes longer than the
// data, so that the distinct A rows one operand read fetches (hi and lo of
// every batch row, same k chunk) start in different LDS banks.
constexpr int kLatRow = 272;                       // int8 hi or lo row
constexpr int kLatRowBF = 528;                     // bf16 row
constexpr int kOffLat = 2048;                      // int8 [kMaxB][2][kLatRow] or bf16 [kMaxB][kLatRowBF]
constexpr int kOffH = kOffLat + kMaxB * 2 * kLatRow;  // float [kMaxB][256]
static_assert(kMaxB * kLatRowBF <= kMaxB * 2 * kLatRow, "bf16 rows fit the latent region");
static_assert(kOffH + 4 * kR <= 12288, "one batch row's h below the staged E rows");
static_assert(kOffH + 4 * kR * kMaxB <= lse_lds_offset(kHeadRecurrent, 0, 2), "h below the lse pairs");
constexpr int kOffAt = 32768;                      // recurrent: A bf16 as [k/8][256 j][8]
constexpr int kOffRecRows = 12288;                 // recurrent, one batch row: staged fp32 E rows [kGroups]
constexpr int kRecRowBytes = kR * 4;


#ifndef WTS_PIN_FULL
#define WTS_PIN_FULL 7
#endif
#ifndef WTS_LDS_RING_1
#define WTS_LDS_RING_1 8
#endif
#ifndef WTS_LDS_RING_2
#define WTS_LDS_RING_2 4
#endif
#ifndef WTS_LDS_RING_4
#define WTS_LDS_RING_4 2
#endif

// Raw buffer resource over [p, p + bytes): loads at byte offsets >= bytes
// return 0.  Word 3 as for untyped loads on gfx9 (32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ v4i mma(const v4i& a, const v4i& b, const v4i& c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mma(const v4i& a, const v4i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                 __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}
template <int WT> struct AccT { typedef v4i T; };
template <> struct AccT<1> { typedef v4f T; };

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long k, int m) {
  const unsigned lo = __shfl_xor((unsigned)k, m, 64);
  const unsigned hi = __shfl_xor((unsigned)(k >> 32), m, 64);
  return ((unsigned long long)hi << 32) | lo;
}

// Per-lane roles.  The MFMA result puts latent row 4q + j (q = lane / 16,
// j = 0..3) of vocabulary column n = lane % 16 in register j.  A lane's
// A-operand row is n.
template <int WT, int BB>
struct Roles {
  using Gm = Geo<WT, BB>;
  int lane, n, q, aslot, aw, cslot, cw0;
  __device__ __forceinline__ explicit Roles(int l) {
    lane = l;
    n = l & 15;
    q = l >> 4;
    aslot = n / Gm::RPS;
    aw = n % Gm::RPS;
    cslot = (4 * q) / Gm::RPS;
    cw0 = (4 * q) % Gm::RPS;
  }
  // batch row of result entry e of M block m (int8: registers 2e (hi), 2e+1 (lo))
  __device__ __forceinline__ int bent(int m, int e) const {
    return WT == 0 ? (m * Gm::RPS + cw0) / 2 + e : m * Gm::RPS + cw0 + e;
  }
  // batch row and hi/lo half of this lane's A-operand row in M block m
  __device__ __forceinline__ int arow_b(int m) const { return (m * Gm::RPS + aw) / Gm::LPB; }
  __device__ __forceinline__ int arow_hl(int m) const { return (m * Gm::RPS + aw) % Gm::LPB; }
};

// ---- workgroup-local selection keys ----
// Inside a workgroup a key orders (score, -row) with the row counted from the
// workgroup's first vocabulary row: T=0 uses 32 bits (a 16-bit order code of
// the bf16 logit, 16-bit row), T=1 64 bits (32-bit order of the fp32 score).
// 0 means "no candidate".  -0 ranks equal to +0.
template <int TEMP> struct LKey { typedef uint32_t T; };
template <> struct LKey<1> { typedef unsigned long long T; };
__device__ __forceinline__ uint32_t ord32(uint32_t b) {
  b = (b == 0x80000000u) ? 0u : b;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ uint32_t kmax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ unsigned long long kmax(unsigned long long a, unsigned long long b) { return a > b ? a : b; }

// Workgroup-local key -> device-wide key (same layout as sel_key: an order
// code of the score in bits 49..18, 0x3FFFF - v in bits 17..0).  T=0 keys of
// all workgroups come through the same code, so only their ranking matters.
__device__ __forceinline__ unsigned long long global_key(uint32_t k, int row0) {
  if (k == 0u) return 0ull;
  const uint32_t o16 = k >> 16;
  const uint32_t o32 = (o16 << 16) | ((o16 & 0x8000u) ? 0u : 0xFFFFu);  // widened, still monotone
  const uint32_t v = (uint32_t)row0 + (0xFFFFu - (k & 0xFFFFu));
  return ((unsigned long long)o32 << 18) | (unsigned long long)(0x3FFFFu - v);
}
__device__ __forceinline__ unsigned long long global_key(unsigned long long k, int row0) {
  if (k == 0ull) return 0ull;
  const uint32_t o32 = (uint32_t)(k >> 16);
  const uint32_t v = (uint32_t)row0 + (0xFFFFu - (uint32_t)(k & 0xFFFFu));
  return ((unsigned long long)o32 << 18) | (unsigned long long)(0x3FFFFu - v);
}

// Max over the 16 lanes of each DPP row (butterfly of quad and mirror moves).
#define WTS_DPP(x, c) ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)(x), (c), 0xF, 0xF, false))
__device__ __forceinline__ uint32_t row_max(uint32_t x) {
  x = kmax(x, WTS_DPP(x, 0xB1));   // quad_perm [1,0,3,2]
  x = kmax(x, WTS_DPP(x, 0x4E));   // quad_perm [2,3,0,1]
  x = kmax(x, WTS_DPP(x, 0x141));  // row_half_mirror
  x = kmax(x, WTS_DPP(x, 0x140));  // row_mirror
  return x;
}
__device__ __forceinline__ unsigned long long row_max(unsigned long long x) {
#define WTS_DPP64(x, c) \
  (((unsigned long long)WTS_DPP((uint32_t)((x) >> 32), (c)) << 32) | WTS_DPP((uint32_t)(x), (c)))
  x = kmax(x, WTS_DPP64(x, 0xB1));
  x = kmax(x, WTS_DPP64(x, 0x4E));
  x = kmax(x, WTS_DPP64(x, 0x141));
  x = kmax(x, WTS_DPP64(x, 0x140));
#undef WTS_DPP64
  return x;
}
// Max over each DPP row of a T=1 local key (32-bit score order << 16 | 16-bit
// row field): the score order first, then the row field among the lanes that
// hold that order.  Two 32-bit butterflies instead of one on 64 bits.
__device__ __forceinline__ unsigned long long row_max_key48(unsigned long long x) {
  const uint32_t hi = (uint32_t)(x >> 16);
  const uint32_t mh = row_max(hi);
  const uint32_t ml = row_max(hi == mh ? (uint32_t)(x & 0xFFFFu) : 0u);
  return ((unsigned long long)mh << 16) | ml;
}
__device__ __forceinline__ uint32_t readlane(uint32_t x, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, l);
}
__device__ __forceinline__ unsigned long long readlane(unsigned long long x, int l) {
  return ((unsigned long long)readlane((uint32_t)(x >> 32), l) << 32) | readlane((uint32_t)x, l);
}

// 1 KiB of zeros in device memory: the A-operand source of the lanes whose
// A row holds no batch row of this walk.
__device__ __attribute__((aligned(64))) int4 g_zero_page[64];

// Latent of this step as MFMA A operands: lane l holds A row (l & 15) -- the
// latent row (batch row, and hi or lo half for int8) of result row
// (l & 15) % RPS -- and k chunk (l >> 4) of every 64-k (int8) or 32-k (bf16)
// step.  Every slot of RPS A rows holds the same latent rows, so one operand
// serves the S tiles of a group, each with its own accumulator.
template <int WT, int BB, int HEAD>
__device__ __forceinline__ void load_latent(const WalkArgs& a, const Roles<WT, BB>& ro, const int* sx,
                                            const char* lds, v4i (&lat)[Geo<WT, BB>::NM][Geo<WT, BB>::CH]) {
  using Gm = Geo<WT, BB>;
#pragma unroll
  for (int m = 0; m < Gm::NM; ++m) {
    const int b = ro.arow_b(m);
    const bool ok = b < a.B;
    const int hl = ro.arow_hl(m);
    if (HEAD == kHeadMarkov) {
      const int x = ok ? sx[b] : 0;
      const v4i* src = WT == 0 ? (const v4i*)(a.Eq + (size_t)x * 512 + hl * 256 + ro.q * 16)
                               : (const v4i*)(a.Eb + (size_t)x * kR + ro.q * 8);
      const v4i* p = ok ? src : (const v4i*)g_zero_page;
#pragma unroll
      for (int c = 0; c < Gm::CH; ++c) lat[m][c] = p[c * 4];
    } else {
      const char* src = WT == 0 ? lds + kOffLat + (b * 2 + hl) * kLatRow + ro.q * 16
                                : lds + kOffLat + b * kLatRowBF + ro.q * 16;
#pragma unroll
      for (int c = 0; c < Gm::CH; ++c) lat[m][c] = ok ? *(const v4i*)(src + c * 64) : v4i{0, 0, 0, 0};
    }
  }
}

// Same A operands as load_latent, from the candidate rows staged in LDS.
template <int WT, int BB>
__device__ __forceinline__ void load_latent_staged(const WalkArgs& a, const Roles<WT, BB>& ro, const char* lds,
                                                   v4i (&lat)[Geo<WT, BB>::NM][Geo<WT, BB>::CH]) {
  using Gm = Geo<WT, BB>;
#pragma unroll
  for (int m = 0; m < Gm::NM; ++m) {
    const int b = ro.arow_b(m);
    const bool ok = b < a.B;
    const int slot = ok ? ((const int*)(lds + kOffWin))[b] : 0;
    const char* src = lds + kOffRows + slot * kRowBytes + ro.arow_hl(m) * kLoOff + ro.q * 16;
    const char* p = ok ? src : lds + kOffZero;
#pragma unroll
    for (int c = 0; c < Gm::CH; ++c) lat[m][c] = *(const v4i*)(p + c * 64);
  }
}

// Result of this lane's tile in a group: accumulator s holds tile s of the
// group in every lane; the lanes of result slot s (l >> 4 in slot s) take it.
// (Bit masks rather than selects, so that the accumulators stay in registers
// instead of becoming a dynamically indexed array.)
template <int S, class AT>
__device__ __forceinline__ AT pick_slot(const AT (&acc)[S], int cslot) {
  v4i r = {0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int mask = -(int)(cslot == s);
    r |= __builtin_bit_cast(v4i, acc[s]) & v4i{mask, mask, mask, mask};
  }
  return __builtin_bit_cast(AT, r);
}

// ---- per-step log normaliser of the logits (optional output) ----
// ln sum_v exp(l_v) is accumulated as (max, sum) pairs in base 2: the pair
// (m, s) stands for s * 2^m.  Each lane folds its logits into running pairs
// (one per result entry), the pairs are merged across lanes, waves and
// workgroups, and the merged pair of each (row, step) becomes (m + log2 s) ln 2.
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2f = 0.69314718055994531f;
constexpr float kLseNone = -3.0e38f;  // max of an empty pair; 2^(kLseNone - m) is 0

struct LsePair {
  float m, s;
};
__device__ __forceinline__ LsePair lse_merge(LsePair x, LsePair y) {
  const float M = fmaxf(x.m, y.m);
  return {M, x.s * __builtin_amdgcn_exp2f(x.m - M) + y.s * __builtin_amdgcn_exp2f(y.m - M)};
}
__device__ __forceinline__ LsePair lse_xor(LsePair p, int o) {
  return lse_merge(p, {__shfl_xor(p.m, o), __shfl_xor(p.s, o)});
}
// Merge over the 16 lanes of each DPP row (the butterfly of row_max).
#define WTS_DPPF(x, c) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), (c), 0xF, 0xF, false))
__device__ __forceinline__ LsePair lse_row_merge(LsePair p) {
  p = lse_merge(p, {WTS_DPPF(p.m, 0xB1), WTS_DPPF(p.s, 0xB1)});
  p = lse_merge(p, {WTS_DPPF(p.m, 0x4E), WTS_DPPF(p.s, 0x4E)});
  p = lse_merge(p, {WTS_DPPF(p.m, 0x141), WTS_DPPF(p.s, 0x141)});
  p = lse_merge(p, {WTS_DPPF(p.m, 0x140), WTS_DPPF(p.s, 0x140)});
  return p;
}
#undef WTS_DPPF

template <int NM, int NE, bool LS>
struct LseAcc {
  float m[NM][NE], s[NM][NE];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < NM; ++i)
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        m[i][e] = kLseNone;
        s[i][e] = 0.0f;
      }
  }
  // fold logit l of a valid (row, batch) pair into entry (i, e)
  __device__ __forceinline__ void add(int i, int e, float l, bool ok) {
    const float y = l * kLog2e;
    const float M = ok ? fmaxf(m[i][e], y) : m[i][e];
    s[i][e] = s[i][e] * __builtin_amdgcn_exp2f(m[i][e] - M) + (ok ? __builtin_amdgcn_exp2f(y - M) : 0.0f);
    m[i][e] = M;
  }
};
template <int NM, int NE>
struct LseAcc<NM, NE, false> {
  __device__ __forceinline__ void init() {}
  __device__ __forceinline__ void add(int, int, float, bool) {}
};

// Fig. 7 epilogue for the result entries of one M block, then the local
// selection (Fig. 8 step 1): logit = bf16(((acc_hi s_hi + acc_lo s_lo) s_w) +
// base) for int8 W, bf16(acc + base) for bf16 W; score = logit (T=0) or
// logit + Gumbel noise (T=1); keep the largest key per batch entry.
// Branch-free: lanes without a valid (row, batch) pair contribute key 0.
// With NZ, T=1 noise comes from LDS (computed one step ahead):
// noise[b * a.noise_stride + (v - row0)], row0 = the workgroup's first row.
// With LS, the logit also enters the running log-sum-exp pairs.
// With BS, the logit is written by a buffer store whose offset lies past the
// end when nothing is to be written (such stores are dropped), so the epilogue
// has no branch and the scheduler can interleave it with the next group's MFMAs.
template <int WT, int BB, int TEMP, bool NZ, bool LS, bool GP = false, bool BS = false>
__device__ __forceinline__ void epilogue(const WalkArgs& a, const Roles<WT, BB>& ro, int t, int m,
                                         const typename AccT<WT>::T& acc, int v, uint32_t lrow, bool ok,
                                         float sw, const uint16_t (&bv)[Geo<WT, BB>::NE],
                                         const float (&shi)[Geo<WT, BB>::NM][Geo<WT, BB>::NE],
                                         typename LKey<TEMP>::T (&best)[Geo<WT, BB>::NM][Geo<WT, BB>::NE],
                                         LseAcc<Geo<WT, BB>::NM, Geo<WT, BB>::NE, LS>& ls,
                                         const float* noise, int row0, const float* gpre = nullptr) {
  using Gm = Geo<WT, BB>;
#pragma unroll
  for (int e = 0; e < Gm::NE; ++e) {
    const int b = ro.bent(m, e);
    if (b >= BB) continue;  // compile-time: entry unused by this batch bucket
    const bool okb = ok && b < a.B;
    float z;
    if (WT == 0) {
      const float zh = (float)acc[2 * e] * shi[m][e];
      const float zl = (float)acc[2 * e + 1] * (shi[m][e] * 0.00390625f);
      z = zh + zl;
      z = z * sw;
    } else {
      z = acc[e];
    }
    z = z + bf16_f32((uint32_t)bv[e]);
    // bf16 rounding to nearest even: the upper half of r is the logit
    const uint32_t zb = __float_as_uint(z);
    const uint32_t r = zb + 0x7FFFu + ((zb >> 16) & 1u);
    if constexpr (BS) {
      // the logits have the shape of the base logits: the same 32-bit byte offsets
      const uint32_t off = okb ? 2u * (((uint32_t)b * (uint32_t)a.gamma + (uint32_t)t) * (uint32_t)a.V + (uint32_t)v)
                               : 0xFFFFFFFEu;
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(r >> 16),
                                            buf_rsrc(a.logits, a.logits != nullptr ? a.base_bytes : 0u), off, 0, 0);
    } else if (a.logits != nullptr) {  // uniform: skipped entirely when logits are not requested
      if (okb) a.logits[((size_t)b * a.gamma + t) * a.V + v] = (uint16_t)(r >> 16);
    }
    const float lf = __uint_as_float(r & 0xFFFF0000u);  // the logit, widened exactly
    ls.add(m, e, lf, okb);
    typename LKey<TEMP>::T k;
    if (TEMP == 0) {
      // order of the bf16 logit in the upper half: positives above negatives,
      // negatives complemented and moved up by one so that -0 ties with +0
      // (the ranking of the rounded logit with -0 taken as +0), row field below
      const uint32_t sg = (uint32_t)((int32_t)r >> 31);
      const uint32_t o = (r ^ (sg | 0x80000000u)) + (sg & 0x10000u);
      k = (o & 0xFFFF0000u) | lrow;
    } else {
      // lanes without a valid pair read the buffer's first element
      // GP: this entry's noise was read from LDS at the start of the step
      const float g = GP   ? gpre[e]
                      : NZ ? noise[okb ? b * a.noise_stride + (v - row0) : 0]
                           : gumbel(a.seed_lo, a.seed_hi, b, a.step_offset + t, v);
      const float sc = lf + g;
      k = ((unsigned long long)ord32(__float_as_uint(sc)) << 16) | lrow;
    }
    best[m][e] = kmax(best[m][e], okb ? k : (typename LKey<TEMP>::T)0);
  }
}

// Base logits of one result entry set (bf16 bits), zero where unused.  The
// row index is made opaque so that the per-lane addresses are recomputed at
// every step instead of being kept in registers for the whole walk.
//
// Buffer loads: element (b, t, v) sits at byte 2 ((b gamma + t) V + v) of
// the base logits, and the batch row of entry e of M block m is the lane's
// first row lb = bent(0, 0) plus m RPS / LPB + e, so one offset per call
// and one add per entry address every entry.  Every lane loads, so the loads
// are straight-line code and nothing waits for them before their use; a
// buffer load past the end (a batch row >= B) returns 0, and the epilogue
// drops the pairs that do not exist (`ok` false, or a row >= B).
template <int WT, int BB>
__device__ __forceinline__ void load_base(const WalkArgs& a, const Roles<WT, BB>& ro, int t, int m,
                                          int v, bool ok, uint16_t (&bv)[Geo<WT, BB>::NE]) {
  using Gm = Geo<WT, BB>;
  (void)ok;
  int lb = ro.bent(0, 0);
  asm volatile("" : "+v"(v), "+v"(lb));
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(a.base, a.base_bytes);
  const uint32_t plane = (uint32_t)a.gamma * (uint32_t)a.V;  // elements per batch row
  const uint32_t off = 2u * ((uint32_t)lb * plane + (uint32_t)t * (uint32_t)a.V + (uint32_t)v);
#pragma unroll
  for (int e = 0; e < Gm::NE; ++e) {
    const int u = m * Gm::RPS / Gm::LPB + e;  // batch row bent(m, e) - lb, known at compile time
    if (u >= BB) {  // no lane's entry e is a row of this batch bucket
      bv[e] = 0;
      continue;
    }
    // unconditional: a lane whose row is >= B reads past the buffer, i.e. 0
    bv[e] = __builtin_amdgcn_raw_buffer_load_b16(rs, off + 2u * (uint32_t)u * plane, 0, 0);
  }
}

// One W tile that is not register-resident, with its row scale and base
// logits, as loaded one tile ahead of its use.
template <int WT, int BB>
struct TileBuf {
  v4i w[Geo<WT, BB>::CH];
  float sw;
  uint16_t bv[Geo<WT, BB>::NM][Geo<WT, BB>::NE];  // bf16 bits, widened where used
};

// Load wave-local tile i (from LDS for i < i0 + nlds, else from memory) for
// step t.  Lanes whose C-slot is 0 own the tile's vocabulary rows.
template <int WT, int BB, int NWV>
__device__ __forceinline__ void fetch_tile(const WalkArgs& a, const Roles<WT, BB>& ro, int t, int tb, int w,
                                           int i, int i0, int nlds, const char* ldsw, TileBuf<WT, BB>& d) {
  using Gm = Geo<WT, BB>;
  constexpr int TB = WT == 0 ? kTileBytesI8 : kTileBytesBF;
  const int tile = tb + w + NWV * i;
  // LDS and global pointers kept apart, so that the two branches stay LDS and
  // global loads (one merged generic load would count against both wait
  // counters and make every wait conservative)
  typedef const __attribute__((address_space(3))) char lds_char;
  typedef const __attribute__((address_space(1))) v4i glb_v4i;
  if (i < i0 + nlds) {
    lds_char* p = (lds_char*)(ldsw + (size_t)(i - i0) * TB + ro.lane * 16);
#pragma unroll
    for (int c = 0; c < Gm::CH; ++c) d.w[c] = *(const __attribute__((address_space(3))) v4i*)(p + c * 1024);
  } else {
    glb_v4i* p = (glb_v4i*)((const v4i*)a.Wp + (size_t)tile * Gm::CH * 64 + ro.lane);
#pragma unroll
    for (int c = 0; c < Gm::CH; ++c) d.w[c] = p[c * 64];
  }
  const int v = tile * kTileRows + ro.n;
  const bool ok = ro.cslot == 0 && v < a.V;
  // every lane loads (see load_base); rows past the padded scales read 0
  d.sw = WT == 0 ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                  buf_rsrc(a.sw, (uint32_t)a.tiles * kTileRows * 4u), 4u * (uint32_t)v, 0, 0))
                 : 0.0f;
#pragma unroll
  for (int m = 0; m < Gm::NM; ++m) load_base<WT, BB>(a, ro, t, m, v, ok, d.bv[m]);
}

// Tiles [i0, nw) of wave w, one tile per MFMA group (slot 0), D - 1 tiles of
// prefetch (D buffers; D = 1: one buffer and a copy).  `cur` holds tile i0 of
// this step, loaded before the step began (a copy: its buffer is reused for
// the tiles after it).
template <int WT, int BB, int TEMP, int NWV, bool NZ, bool LS, int D>
__device__ __forceinline__ void stream_tiles(const WalkArgs& a, const Roles<WT, BB>& ro, int t, int tb,
                                             int w, int i0, int nlds, int nw, const char* ldsw,
                                             TileBuf<WT, BB> cur,
                                             const v4i (&lat)[Geo<WT, BB>::NM][Geo<WT, BB>::CH],
                                             const float (&shi)[Geo<WT, BB>::NM][Geo<WT, BB>::NE],
                                             typename LKey<TEMP>::T (&best)[Geo<WT, BB>::NM][Geo<WT, BB>::NE],
                                             LseAcc<Geo<WT, BB>::NM, Geo<WT, BB>::NE, LS>& ls,
                                             const float* noise) {
  const int row0 = tb * kTileRows;
  using Gm = Geo<WT, BB>;
  using AT = typename AccT<WT>::T;
  auto compute = [&](const TileBuf<WT, BB>& cur, int i) {
    const int tile = tb + w + NWV * i;
    const int v = tile * kTileRows + ro.n;
    const bool ok = ro.cslot == 0 && v < a.V;
    const uint32_t lrow = 0xFFFFu - (uint32_t)((tile - tb) * kTileRows + ro.n);
#pragma unroll
    for (int m = 0; m < Gm::NM; ++m) {
      AT acc = {0, 0, 0, 0}, acc2 = {0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < Gm::CH; ++c) {
        if (WT == 0 && (c & 1)) acc2 = mma(lat[m][c], cur.w[c], acc2);
        else acc = mma(lat[m][c], cur.w[c], acc);
      }
      if (WT == 0) acc = acc + acc2;
      epilogue<WT, BB, TEMP, NZ, LS>(a, ro, t, m, acc, v, lrow, ok, cur.sw, cur.bv[m], shi, best, ls, noise, row0);
    }
  };
  static_assert(D >= 1 && D <= 3, "one, two or three tile buffers");
  if constexpr (D == 3) {
    // Three buffers in turn, two tiles in flight while one is computed.
    TileBuf<WT, BB> b1, b2;
    if (i0 + 1 < nw) fetch_tile<WT, BB, NWV>(a, ro, t, tb, w, i0 + 1, i0, nlds, ldsw, b1);
    for (int i = i0; i < nw; i += 3) {
      if (i + 2 < nw) fetch_tile<WT, BB, NWV>(a, ro, t, tb, w, i + 2, i0, nlds, ldsw, b2);
      compute(cur, i);
      if (i + 1 >= nw) break;
      if (i + 3 < nw) fetch_tile<WT, BB, NWV>(a, ro, t, tb, w, i + 3, i0, nlds, ldsw, cur);
      compute(b1, i + 1);
      if (i + 2 >= nw) break;
      if (i + 4 < nw) fetch_tile<WT, BB, NWV>(a, ro, t, tb, w, i + 4, i0, nlds, ldsw, b1);
      compute(b2, i + 2);
    }
  } else if constexpr (D == 2) {
    // Two buffers used in turn: the next tile's loads go into the buffer that
    // is not being computed, and nothing is copied from a buffer whose loads
    // are still in flight (a copy would make the wave wait for them at once).
    TileBuf<WT, BB> b1;
    for (int i = i0; i < nw; i += 2) {
      if (i + 1 < nw) fetch_tile<WT, BB, NWV>(a, ro, t, tb, w, i + 1, i0, nlds, ldsw, b1);
      compute(cur, i);
      if (i + 1 >= nw) break;
      if (i + 2 < nw) fetch_tile<WT, BB, NWV>(a, ro, t, tb, w, i + 2, i0, nlds, ldsw, cur);
      compute(b1, i + 1);
    }
  } else {
    // one buffer and a copy (kernels without the registers for two)
    for (int i = i0; i < nw; ++i) {
      TileBuf<WT, BB> nxt;
      if (i + 1 < nw) fetch_tile<WT, BB, NWV>(a, ro, t, tb, w, i + 1, i0, nlds, ldsw, nxt);
      compute(cur, i);
      if (i + 1 < nw) cur = nxt;
    }
  }
}

// Wave-level reduction of the keys (Fig. 8 step 2): DPP maximum inside each
// 16-lane row, then the four rows' maxima per batch row via readlane; lane 0
// writes red[w][b] for b < BB.
template <int WT, int BB, int TEMP>
__device__ __forceinline__ void reduce_to_lds(const Roles<WT, BB>& ro, int w,
                                              typename LKey<TEMP>::T (&best)[Geo<WT, BB>::NM][Geo<WT, BB>::NE],
                                              unsigned long long* red) {
  using Gm = Geo<WT, BB>;
  using K = typename LKey<TEMP>::T;
  K acc_b[BB];
#pragma unroll
  for (int b = 0; b < BB; ++b) acc_b[b] = 0;
#pragma unroll
  for (int m = 0; m < Gm::NM; ++m)
#pragma unroll
    for (int e = 0; e < Gm::NE; ++e) {
      K k;
      if constexpr (TEMP == 1) k = row_max_key48(best[m][e]);
      else k = row_max(best[m][e]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cw0 = (4 * q) % Gm::RPS;
        const int b = WT == 0 ? (m * Gm::RPS + cw0) / 2 + e : m * Gm::RPS + cw0 + e;
        if (b < BB) acc_b[b] = kmax(acc_b[b], readlane(k, 16 * q));
      }
    }
  if (ro.lane == 0) {
#pragma unroll
    for (int b = 0; b < BB; ++b) red[w * kMaxB + b] = (unsigned long long)acc_b[b];
  }
}

// Whether result entry e of M block m holds a batch row of the bucket for
// some lane (the four 16-lane rows map to batch rows as in reduce_to_lds).
template <int WT, int BB>
__device__ constexpr bool entry_used(int m, int e) {
  using Gm = Geo<WT, BB>;
  bool used = false;
  for (int q = 0; q < 4; ++q)
    used = used || (WT == 0 ? (m * Gm::RPS + (4 * q) % Gm::RPS) / 2 + e : m * Gm::RPS + (4 * q) % Gm::RPS + e) < BB;
  return used;
}

// Log-sum-exp pairs of one wave: merged inside each 16-lane row (DPP), then
// the four rows per batch row (same mapping as the keys); lane 0 writes
// lred[w][b] for b < BB.
template <int WT, int BB, bool LS>
__device__ __forceinline__ void lse_reduce_to_lds(const Roles<WT, BB>& ro, int w,
                                                  const LseAcc<Geo<WT, BB>::NM, Geo<WT, BB>::NE, LS>& ls,
                                                  float2* lred) {
  if constexpr (LS) {
    using Gm = Geo<WT, BB>;
    LsePair acc_b[BB];
#pragma unroll
    for (int b = 0; b < BB; ++b) acc_b[b] = {kLseNone, 0.0f};
#pragma unroll
    for (int m = 0; m < Gm::NM; ++m)
#pragma unroll
      for (int e = 0; e < Gm::NE; ++e) {
        if (!entry_used<WT, BB>(m, e)) continue;  // compile-time: entry unused by this batch bucket
        const LsePair p = lse_row_merge({ls.m[m][e], ls.s[m][e]});
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cw0 = (4 * q) % Gm::RPS;
          const int b = WT == 0 ? (m * Gm::RPS + cw0) / 2 + e : m * Gm::RPS + cw0 + e;
          if (b < BB)
            acc_b[b] = lse_merge(acc_b[b], {__int_as_float(__builtin_amdgcn_readlane(__float_as_int(p.m), 16 * q)),
                                            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p.s), 16 * q))});
        }
      }
    if (ro.lane == 0) {
#pragma unroll
      for (int b = 0; b < BB; ++b) lred[w * kMaxB + b] = make_float2(acc_b[b].m, acc_b[b].s);
    }
  }
}

// The workgroup's pair of each batch row (lanes b < B of one wave) to
// lse_part[b][t][g] of a grid of G workgroups.
__device__ __forceinline__ void lse_store_partial(const WalkArgs& a, const float2* lred, int nw, int t, int g,
                                                  int G, int lane) {
  if (lane < a.B) {
    LsePair p = {kLseNone, 0.0f};
    for (int ww = 0; ww < nw; ++ww) {
      const float2 q = lred[ww * kMaxB + lane];
      p = lse_merge(p, {q.x, q.y});
    }
    ((float2*)a.lse_part)[((size_t)lane * a.gamma + t) * G + g] = make_float2(p.m, p.s);
  }
}

// The exchange wave's raw pairs, handed to another wave through LDS
// (lraw[entry][lane]) so that the exchange does not wait for their merge.
template <int WT, int BB, bool LS>
__device__ __forceinline__ void lse_stash(const Roles<WT, BB>& ro,
                                          const LseAcc<Geo<WT, BB>::NM, Geo<WT, BB>::NE, LS>& ls, float2* lraw) {
  if constexpr (LS) {
    using Gm = Geo<WT, BB>;
#pragma unroll
    for (int m = 0; m < Gm::NM; ++m)
#pragma unroll
      for (int e = 0; e < Gm::NE; ++e)
        if (entry_used<WT, BB>(m, e)) lraw[(m * Gm::NE + e) * 64 + ro.lane] = make_float2(ls.m[m][e], ls.s[m][e]);
  }
}

// Per-step pairs of the workgroup while wave 0 runs the exchange: waves
// 1..NW-1 merge their own pairs (the last of them also wave 0's stashed
// pairs); the last wave to finish, found with an LDS counter, merges the
// waves' pairs and stores the workgroup's pair of every batch row.
template <int WT, int BB, int NW, bool LS>
__device__ __forceinline__ void lse_workgroup(const WalkArgs& a, const Roles<WT, BB>& ro, int w,
                                              const LseAcc<Geo<WT, BB>::NM, Geo<WT, BB>::NE, LS>& ls,
                                              float2* lred, const float2* lraw, int* cnt, int t, int g, int G) {
  if constexpr (LS) {
    using Gm = Geo<WT, BB>;
    lse_reduce_to_lds<WT, BB, LS>(ro, w, ls, lred);
    if (w == NW - 1) {
      LseAcc<Gm::NM, Gm::NE, LS> l0;
      l0.init();
#pragma unroll
      for (int m = 0; m < Gm::NM; ++m)
#pragma unroll
        for (int e = 0; e < Gm::NE; ++e)
          if (entry_used<WT, BB>(m, e)) {
            const float2 q = lraw[(m * Gm::NE + e) * 64 + ro.lane];
            l0.m[m][e] = q.x;
            l0.s[m][e] = q.y;
          }
      lse_reduce_to_lds<WT, BB, LS>(ro, 0, l0, lred);
    }
    int last = 0;
    if (ro.lane == 0)
      last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP) == NW - 2;
    if (__builtin_amdgcn_readfirstlane(last)) {
      lse_store_partial(a, lred, NW, t, g, G, ro.lane);
      if (ro.lane == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
}

// Merge the partials of all G workgroups of every (row, step) into lse:
// one wave per (row, step), launched after the walk on the same stream.
constexpr int kLseWaves = 4;
__global__ __launch_bounds__(kLseWaves * 64) void lse_kernel(WalkArgs a, int G) {
  const int lane = threadIdx.x & 63;
  const int p = blockIdx.x * kLseWaves + (threadIdx.x >> 6);
  if (p >= a.B * a.gamma) return;
  LsePair acc = {kLseNone, 0.0f};
  const float2* src = (const float2*)a.lse_part + (size_t)p * G;
  for (int i = lane; i < G; i += 64) {
    const float2 q = src[i];
    acc = lse_merge(acc, {q.x, q.y});
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) acc = lse_xor(acc, o);
  if (lane == 0) a.lse[p] = (acc.m + log2f(acc.s)) * kLn2f;
}

__device__ __forceinline__ void latch_error(Ctrl* ctrl, unsigned code) {
  atomicCAS(&ctrl->err, 0u, code);
}

// Parity of the walk that reads it (every launch of one walk reads the same
// epoch: the walk advances it only at its very end).
__device__ __forceinline__ int walk_parity(Ctrl* ctrl) {
  // one value for the whole wave, held in a scalar register
  return __builtin_amdgcn_readfirstlane(
      (int)(__hip_atomic_load(&ctrl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 1u));
}
__device__ __forceinline__ void advance_epoch(Ctrl* ctrl) {
  __hip_atomic_fetch_add(&ctrl->epoch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long ld_agent(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Signalling inside one XCD through its shared L2: a plain store (the CU's
// L1 writes through to the L2) and a load with the non-temporal bit (NT=1)
// at the default scope.  For such a load the vector L1 applies its streaming
// policy and keeps no copy of the line, so every poll is served by the L2,
// where the other workgroups of the XCD store.  About 0.28 us one way on
// MI355X, against 0.47 us for the device-scope pair above, which bypasses the
// L2.  (Were a polled line kept in L1, the poll would never see the new key,
// and the watchdog would latch a time-out rather than a wrong token.)
__device__ __forceinline__ void st_xcd(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// N such loads in flight at once, then one wait.
template <int N>
__device__ __forceinline__ void ld_xcd(const unsigned long long* const (&p)[N], unsigned long long (&v)[N]) {
  static_assert(N == 1 || N == 2 || N == 4, "1, 2 or 4 loads");
  if constexpr (N == 1) {
    asm volatile("global_load_dwordx2 %0, %1, off nt\n\ts_waitcnt vmcnt(0)" : "=v"(v[0]) : "v"(p[0]) : "memory");
  } else if constexpr (N == 2) {
    asm volatile(
        "global_load_dwordx2 %0, %2, off nt\n\tglobal_load_dwordx2 %1, %3, off nt\n\ts_waitcnt vmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1])
        : "v"(p[0]), "v"(p[1])
        : "memory");
  } else {
    asm volatile(
        "global_load_dwordx2 %0, %4, off nt\n\tglobal_load_dwordx2 %1, %5, off nt\n\t"
        "global_load_dwordx2 %2, %6, off nt\n\tglobal_load_dwordx2 %3, %7, off nt\n\ts_waitcnt vmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3])
        : "memory");
  }
}

// LDS address of a pointer into the workgroup's LDS, for hand-issued LDS
// reads.  The compiler makes every LDS access it emits wait for all
// outstanding global->LDS copies (it cannot tell which bytes they write); a
// polling loop that starts such copies reads its LDS words by hand instead.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Clear the control arrays of the next walk (parity par ^ 1), spread over
// the whole grid.  Nothing in this walk touches them.  OWN_L1: each
// workgroup clears its own first-level lines (the persistent walk, whose
// first level stays inside an XCD); otherwise the grid clears all of them.
template <bool OWN_L1, int NTH = 0, bool PACKED = false>
__device__ __forceinline__ void clear_next_walk(Ctrl* ctrl, int par) {
  const int q = par ^ 1;
  if (OWN_L1 && threadIdx.x < 2 * kMaxB) {
    const int g = blockIdx.x, b = threadIdx.x % kMaxB;
    const int at = PACKED ? ((g % kGroups) * kMaxB + b) * kGroups + g / kGroups : g * kMaxB + b;
    (&ctrl->l1[q][threadIdx.x / kMaxB][0][0])[at] = 0ull;
  }
  const size_t n1 = OWN_L1 ? 0 : sizeof(ctrl->l1[0]) / 8, n2 = sizeof(ctrl->l2[0]) / 8, n3 = sizeof(ctrl->ss[0]) / 8;
  unsigned long long* p1 = &ctrl->l1[q][0][0][0];
  unsigned long long* p2 = &ctrl->l2[q][0][0][0][0];
  unsigned long long* p3 = &ctrl->ss[q][0][0][0];
  // NTH: the block size when known at compile time (blockDim.x is read from
  // the dispatch packet, a memory load)
  const int nth = NTH > 0 ? NTH : (int)blockDim.x;
  const size_t stride = (size_t)gridDim.x * nth;
  for (size_t i = (size_t)blockIdx.x * nth + threadIdx.x; i < n1 + n2 + n3; i += stride) {
    if (i < n1) p1[i] = 0ull;
    else if (i < n1 + n2) p2[i - n1] = 0ull;
    else p3[i - n1 - n2] = 0ull;
  }
}

// Rotation by N lanes inside each 16-lane DPP row (row_ror), 64-bit.
template <int N>
__device__ __forceinline__ unsigned long long row_ror64(unsigned long long x) {
  return ((unsigned long long)WTS_DPP((uint32_t)(x >> 32), 0x120 + N) << 32) | WTS_DPP((uint32_t)x, 0x120 + N);
}

// Maximum over the lanes that hold the same batch row (lane % BB) among the
// first 16 * BB lanes; every lane of those rows ends with its class maximum.
// DPP inside the 16-lane rows (the whole row for BB = 1, rotations by
// multiples of BB otherwise), then across rows.
template <int BB>
__device__ __forceinline__ unsigned long long class_max(unsigned long long x) {
  if constexpr (BB == 1) {
    return row_max(x);  // 16 entries: one row
  } else {
    if constexpr (BB <= 8) x = kmax(x, row_ror64<BB>(x));
    if constexpr (BB <= 4) x = kmax(x, row_ror64<2 * BB>(x));
    if constexpr (BB <= 2) x = kmax(x, row_ror64<4 * BB>(x));
    x = kmax(x, shfl_xor_u64(x, 16));
    if constexpr (BB >= 4) x = kmax(x, shfl_xor_u64(x, 32));
    return x;
  }
}

// Cross-workgroup selection of one step (Fig. 8), one wave per workgroup.
// Every workgroup publishes its local winner key per batch row, tagged with
// the step, in its own line; the first workgroup of each of kGroups groups
// waits for its members' keys and publishes the group maximum in kCopies
// copies; every workgroup waits for the kGroups group maxima in copy
// (g % kCopies) and takes the overall maximum.  Workgroups are dispatched
// round-robin over the XCDs (g % 8 on MI355X; the host checks this at create
// time), so a group (g % kGroups) lies on one XCD and, with xl1, its keys
// travel through that XCD's L2 (st_xcd / ld_xcd); only the group maxima cross
// XCDs (device scope, one copy per XCD).  Without xl1 (the dispatch check
// failed, or the caller asked for it) the first level uses device scope too.
// A stale line never passes for a new one, since every key carries its step.  The keys carry the token, so no other data has to be
// made visible: relaxed loads and stores suffice.  Returns false if the
// watchdog expired.  On return, lanes b < B hold the winning key of row b.
// PACKED: the keys one poll reads share 128-byte lines -- first level
// [group][row][member], second level [copy][row][group] -- instead of one
// line per workgroup and per group.
template <int BB, bool CAND, bool PACKED = false>
__device__ __forceinline__ bool exchange(Ctrl* ctrl, int par, int t, int B, unsigned long long key,
                                         long long timeout, unsigned long long* winner, char* lds, bool xl1) {
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x, G = gridDim.x;
  const unsigned long long want = (unsigned long long)(t + 1);
  const unsigned long long tag = want << kTagShift;
  unsigned long long* L1 = &ctrl->l1[par][t & 1][0][0];
  unsigned long long* L2 = &ctrl->l2[par][t & 1][0][0][0];
  const int grp = g % kGroups;
  // line index of member i's key of row b (group grp), and of group x's maximum of row b in copy c
  auto l1_at = [&](int i, int b) { return PACKED ? (grp * kMaxB + b) * kGroups + i : (grp + kGroups * i) * kMaxB + b; };
  auto l2_at = [&](int c, int x, int b) { return PACKED ? (c * kMaxB + b) * kGroups + x : (c * kGroups + x) * kMaxB + b; };
  if (lane < B) {
    if (xl1) st_xcd(&L1[l1_at(g / kGroups, lane)], tag | key);
    else st_agent(&L1[l1_at(g / kGroups, lane)], tag | key);
  }
  const long long t0 = wall_clock64();
  bool ok_all = true;
  if (g < kGroups) {
    const int nmem = (G - grp + kGroups - 1) / kGroups;  // at most kGroups members (G <= 256)
    // member keys of this lane: entries q = lane + 64 k, member q / BB, row q % BB
    constexpr int NQ = (kGroups * BB + 63) / 64;
    const unsigned long long* pp[NQ];
    bool act[NQ];
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
      const int q = lane + 64 * k, i = q / BB, b = q % BB;
      act[k] = q < nmem * BB && b < B;
      pp[k] = act[k] ? &L1[l1_at(i, b)] : &L1[l1_at(g / kGroups, 0)];  // idle lanes: own key
    }
    unsigned long long best;
    while (true) {
      unsigned long long v[NQ];
      if (xl1) {
        ld_xcd<NQ>(pp, v);
      } else {
#pragma unroll
        for (int k = 0; k < NQ; ++k) v[k] = ld_agent(pp[k]);
      }
      bool ok = true;
      best = 0ull;
#pragma unroll
      for (int k = 0; k < NQ; ++k)
        if (act[k]) {
          ok = ok && (v[k] >> kTagShift) == want;
          best = umax64(best, v[k]);
        }
      if (__all(ok)) break;
      if (wall_clock64() - t0 > timeout) {
        ok_all = false;
        break;
      }
    }
    best = class_max<BB>(best);
    if (ok_all) {
      // after class_max every lane holds the maximum of batch row (lane % BB)
      for (int q = lane; q < kCopies * BB; q += 64) {
        const int r = q / BB, b = q % BB;
        if (b < B) st_agent(&L2[l2_at(r, grp, b)], best);
      }
    }
  }
  const int ngr = G < kGroups ? G : kGroups;
  // group maxima of this lane: entries q = lane + 64 k, group q / BB, row q % BB,
  // all loads of a poll in flight at once
  constexpr int NQ2 = (kGroups * BB + 63) / 64;
  const unsigned long long* p2[NQ2];
  bool act2[NQ2];
#pragma unroll
  for (int k = 0; k < NQ2; ++k) {
    const int q = lane + 64 * k, x = q / BB, b = q % BB;
    act2[k] = q < ngr * BB && b < B;
    p2[k] = &L2[l2_at(g % kCopies, act2[k] ? x : 0, act2[k] ? b : 0)];
  }
  unsigned long long best = 0ull;
  while (ok_all) {
    unsigned long long v[NQ2];
#pragma unroll
    for (int k = 0; k < NQ2; ++k) v[k] = ld_agent(p2[k]);
    bool ok = true;
    best = 0ull;
#pragma unroll
    for (int k = 0; k < NQ2; ++k)
      if (act2[k]) {
        const bool here = (v[k] >> kTagShift) == want;
        ok = ok && here;
        best = umax64(best, v[k]);
        if (CAND && here)  // let wave 1 start staging this candidate's row
          __hip_atomic_store((unsigned long long*)(lds + kOffCand) + lane + 64 * k, v[k], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    if (__all(ok)) break;
    if (wall_clock64() - t0 > timeout) ok_all = false;
  }
  best = class_max<BB>(best);
  *winner = best & kKeyMask;
  if (CAND && lane == 0)
    __hip_atomic_store((int*)(lds + kOffDone), ok_all ? t + 1 : -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return ok_all;
}

// Wave 1 during the exchange of step t (one batch row): as wave 0 publishes
// group maxima in LDS, copy the embedding row of the largest candidate seen
// so far (Markov: hi | lo and s_hi; recurrent: the fp32 row) from memory
// straight into LDS (global_load_lds: no registers, nothing waits for it
// inside the loop).  Every poll reduces all candidates at once (lane c holds
// group c's key), so a new maximum starts its copy one LDS round trip after
// wave 0 stores it; only a candidate larger than all earlier ones can win, so
// the last row copied is the winner's once the exchange is complete.  Then
// record which staged row that is and wait for the copies.  The next step
// builds its latent from LDS.
template <int HEAD, int BB>
__device__ __forceinline__ void stage_rows(const WalkArgs& a, int t, char* lds, long long timeout) {
  static_assert(BB == 1, "one batch row: the group maxima are the lanes of DPP row 0");
  typedef __attribute__((address_space(3))) void lds_void;
  const int lane = threadIdx.x & 63;
  const int ngr = gridDim.x < kGroups ? gridDim.x : kGroups;
  const unsigned long long want = (unsigned long long)(t + 1);
  const bool mine = lane < ngr;  // lane = candidate of group `lane`
  const unsigned long long* cand = (const unsigned long long*)(lds + kOffCand);
  unsigned long long bestk = 0ull;
  int bestc = 0;
  auto stage_new = [&](unsigned long long kl) {
    const unsigned long long k = (mine && (kl >> kTagShift) == want) ? kl : 0ull;
    const unsigned long long m = readlane(row_max(k), 0);  // lanes >= 16 hold no candidate
    if (m <= bestk) return;
    bestk = m;
    bestc = __builtin_ctzll(__ballot(k == m));
    const int v = key_token(m & kKeyMask);
    if (v < 0 || v >= a.V) return;
    if (HEAD == kHeadMarkov) {
      // lane i fills bytes [16 i, 16 i + 16) of the staged row: lanes 0..15
      // the hi half, lanes kLoOff/16.. the lo half
      const int lo = lane - kLoOff / 16;
      if (lane < 16 || (lo >= 0 && lo < 16))
        __builtin_amdgcn_global_load_lds((const void*)(a.Eq + (size_t)v * 512 + (lane < 16 ? lane * 16 : 256 + lo * 16)),
                                         (lds_void*)(lds + kOffRows + bestc * kRowBytes), 16, 0, 0);
      if (lane == 0)
        __builtin_amdgcn_global_load_lds((const void*)(a.Es + v), (lds_void*)(lds + kOffShs + bestc * 4), 4, 0, 0);
    } else {
      // the fp32 row, 16 bytes per lane
      __builtin_amdgcn_global_load_lds((const void*)(a.E + (size_t)v * kR + lane * 4),
                                       (lds_void*)(lds + kOffRecRows + bestc * kRecRowBytes), 16, 0, 0);
    }
  };
  // Every lane reads its candidate word (lanes past the candidates read unused
  // bytes below the rows) and the done flag, with one wait for both.
  const uint32_t a_cand = lds_addr(cand + lane), a_done = lds_addr(lds + kOffDone);
  auto poll = [&](unsigned long long& kl) {
    int dn;
    asm volatile("ds_read_b64 %0, %2\n\tds_read_b32 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(kl), "=&v"(dn)
                 : "v"(a_cand), "v"(a_done)
                 : "memory");
    return __builtin_amdgcn_readfirstlane(dn);
  };
  const long long t0 = wall_clock64();
  for (int it = 1;; ++it) {
    unsigned long long kl;
    const int dn = poll(kl);
    stage_new(kl);
    if (dn == t + 1 || dn == -1) break;
    if ((it & 7) == 0 && wall_clock64() - t0 > timeout) break;  // the watchdog, every 8 polls
  }
  {
    unsigned long long kl;
    poll(kl);
    stage_new(kl);  // candidates published in the last poll
  }
  if (lane == 0) ((int*)(lds + kOffWin))[0] = bestc;
  __builtin_amdgcn_s_waitcnt(0);  // the LDS copies are complete before the workgroup barrier
}

// Recurrent head, first half of a step (Fig. 13): h_{t+1} = tanh(A h_t +
// E[x_t] + c) with the A h_t sums (ascending k) already in racc; then the
// latent rows for the projection (int8 hi/lo + s_hi, or bf16) into LDS.
// staged: E[x_t] is the candidate row staged in LDS during the exchange.
template <int WT, int BB>
__device__ __forceinline__ void recurrent_advance(const WalkArgs& a, int tid, const int* sx, char* lds,
                                                  const float (&racc)[BB], float cj, bool staged) {
  float* h = (float*)(lds + kOffH);
  if (tid >= kThreads - kR) {
    const int j = tid - (kThreads - kR);
#pragma unroll
    for (int b = 0; b < BB; ++b)
      if (b < a.B) {
        const float e = staged ? ((const float*)(lds + kOffRecRows + ((const int*)(lds + kOffWin))[b] *
                                                            kRecRowBytes))[j]
                               : a.E[(size_t)sx[b] * kR + j];
        const float pre = (racc[b] + e) + cj;
        h[b * kR + j] = tanh_p(pre);
      }
  }
  __syncthreads();
  const int w = tid >> 6, lane = tid & 63;
  for (int b = w; b < a.B; b += kWaves) {
    const float4 u4 = *(const float4*)(h + b * kR + lane * 4);
    if (WT == 0) {
      const float u[4] = {u4.x, u4.y, u4.z, u4.w};
      uint32_t hi, lo;
      const float s = quant4(u, &hi, &lo);
      *(uint32_t*)(lds + kOffLat + (b * 2 + 0) * kLatRow + lane * 4) = hi;
      *(uint32_t*)(lds + kOffLat + (b * 2 + 1) * kLatRow + lane * 4) = lo;
      if (lane == 0) ((float*)(lds + kOffShi))[b] = s;
    } else {
      uint16_t* lb = (uint16_t*)(lds + kOffLat + b * kLatRowBF) + lane * 4;
      lb[0] = (uint16_t)bf16_rne(u4.x);
      lb[1] = (uint16_t)bf16_rne(u4.y);
      lb[2] = (uint16_t)bf16_rne(u4.z);
      lb[3] = (uint16_t)bf16_rne(u4.w);
    }
  }
  __syncthreads();
}

// Recurrent head (Fig. 13 gives h = tanh(A h + E[x] + c), no summation
// order): racc[b] = sum_k A[j][k] h[b][k] in binary32 as one chain in
// ascending k from +0, every product and every addition rounded once (no
// fused multiply-add; the build disables contraction).  Thread j owns output
// j.  A lives in LDS as [k/8][j][8] bf16, so thread j reads the eight
// weights of a k-block with one 16-byte load, widened once and used for every
// batch row; h is read as a broadcast.  The chains of the batch rows are
// independent and interleave.
template <int BB>
__device__ __forceinline__ void recurrent_matvec(const WalkArgs& a, int tid, const char* lds, float (&racc)[BB]) {
  if (tid < kThreads - kR) return;
  const int j = tid - (kThreads - kR);
  const uint4* A8 = (const uint4*)(lds + kOffAt);
  const float* h = (const float*)(lds + kOffH);
#pragma unroll
  for (int b = 0; b < BB; ++b) racc[b] = 0.0f;
  // A loads run D k-blocks ahead of the arithmetic
  constexpr int KB = kR / 8, D = 2;
  uint4 wq[D + 1];
#pragma unroll
  for (int d = 0; d < D; ++d) wq[d] = A8[d * kR + j];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    if (kb + D < KB) wq[(kb + D) % (D + 1)] = A8[(kb + D) * kR + j];
    const uint4 w8 = wq[kb % (D + 1)];
    float av[8];
    av[0] = __uint_as_float(w8.x << 16);
    av[1] = __uint_as_float(w8.x & 0xFFFF0000u);
    av[2] = __uint_as_float(w8.y << 16);
    av[3] = __uint_as_float(w8.y & 0xFFFF0000u);
    av[4] = __uint_as_float(w8.z << 16);
    av[5] = __uint_as_float(w8.z & 0xFFFF0000u);
    av[6] = __uint_as_float(w8.w << 16);
    av[7] = __uint_as_float(w8.w & 0xFFFF0000u);
#pragma unroll
    for (int b = 0; b < BB; ++b) {
      if (b >= a.B) continue;
      const float4 h0 = *(const float4*)(h + b * kR + kb * 8);
      const float4 h1 = *(const float4*)(h + b * kR + kb * 8 + 4);
      const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
      float acc = racc[b];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = av[i] * hv[i];
        acc = acc + p;
      }
      racc[b] = acc;
    }
  }
}

// Gumbel noise of step t for every (batch row, vocabulary row) of this
// workgroup into LDS: one Philox4x32-10 call per group of four consecutive
// rows (they share the counter and use its four output words), then
// g = -log(-log U) per word.  count threads share the work; this one is
// number idx among them.
__device__ __forceinline__ void make_noise(const WalkArgs& a, float* noise, int t, int row0, int rows,
                                           int idx, int count) {
  const int quads = rows >> 2;
  const int items = a.B * quads;
  for (int it = idx; it < items; it += count) {
    const int b = it / quads, qd = it - b * quads;
    const int v0 = row0 + 4 * qd;
    uint32_t c0 = (uint32_t)v0 >> 2, c1 = (uint32_t)(a.step_offset + t), c2 = (uint32_t)b, c3 = 0u;
    uint32_t k0 = a.seed_lo, k1 = a.seed_hi;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
      if (r) {
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
      }
      uint32_t hi0, lo0, hi1, lo1;
      mul_wide(0xD2511F53u, c0, hi0, lo0);
      mul_wide(0xCD9E8D57u, c2, hi1, lo1);
      const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
      c0 = n0;
      c1 = lo1;
      c2 = n2;
      c3 = lo0;
    }
    const uint32_t wv[4] = {c0, c1, c2, c3};
    float g[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float u = (float)(2u * (wv[i] >> 9) + 1u) * 5.9604644775390625e-08f;
      g[i] = -log_p(-log_p(u));
    }
    *(float4*)(noise + b * a.noise_stride + 4 * qd) = make_float4(g[0], g[1], g[2], g[3]);
  }
}

// While wave 0 exchanges keys, other waves read one word of every 128-byte
// line of the next step's base logits over this workgroup's rows.  The
// non-register tiles load their base logits only one tile ahead of use; with
// the lines already in the XCD's L2 those loads do not wait for memory.
// At most two lines per thread (a hint: lines past that are not read).
struct BaseTouch {
  uint32_t v[2];
};
__device__ __forceinline__ BaseTouch touch_base(const WalkArgs& a, int t, int row0, int rows, int idx, int count) {
  BaseTouch r{};
  const int r1 = min(row0 + rows, a.V);
  if (r1 > row0) {
    const int nl = (r1 - row0 + 63) / 64 + 1;  // every 64th row (128 bytes apart), then the last row
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int q = idx + k * count;
      if (q < a.B * nl) {
        const int b = q / nl, l = q % nl;
        const int v = l + 1 == nl ? r1 - 1 : row0 + 64 * l;
        r.v[k] = __builtin_amdgcn_raw_buffer_load_b16(
            buf_rsrc(a.base, a.base_bytes), 2u * (((uint32_t)b * (uint32_t)a.gamma + (uint32_t)t) * (uint32_t)a.V + (uint32_t)v),
            0, 0);
      }
    }
  }
  return r;
}
__device__ __forceinline__ void touch_done(const BaseTouch& r, char* lds_dummy) {
  if ((r.v[0] ^ r.v[1]) == 0x9E37u) *lds_dummy = 1;  // keeps the loads; the byte is never read
}

// The whole walk in one persistent launch: grid = one workgroup per CU.
// LS: also the per-step log normaliser of the logits (lse output).
// FULL: the whole shard is on chip (more register tiles, no streaming; each
// wave's LDS tiles follow the previous waves' in LDS).
template <int WT, int BB, int HEAD, int TEMP, bool LS, bool FULL>
__global__ __launch_bounds__(waves_for(HEAD, WT) * 64, 1) void walk_kernel(WalkArgs a) {
  constexpr int NW = waves_for(HEAD, WT);
  constexpr int NT = NW * 64;
  using Gm = Geo<WT, BB, HEAD, FULL, TEMP, LS>;
  using AT = typename AccT<WT>::T;
  constexpr int TB = WT == 0 ? kTileBytesI8 : kTileBytesBF;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  unsigned long long* red = (unsigned long long*)(lds + kOffRed);
  int* sx = (int*)(lds + kOffX);
  int* sflag = (int*)(lds + kOffFlag);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: tile counts and branches stay scalar
  const Roles<WT, BB> ro(tid & 63);
  const int g = blockIdx.x, G = gridDim.x;
  const int tb = (int)((long long)g * a.tiles / G);
  const int te = (int)((long long)(g + 1) * a.tiles / G);
  const int cnt = te - tb;
  const int nw = cnt > w ? (cnt - w + NW - 1) / NW : 0;
  const int nreg = min(nw, a.reg_tiles);
  const int nlds = FULL ? min(nw - nreg, kFullLdsMax) : min(nw - nreg, a.lds_tiles + (w < a.lds_extra ? 1 : 0));
  Ctrl* ctrl = a.ctrl;
  // The walk's epoch and the first state are requested before the shard, so
  // that their latency overlaps the shard load instead of preceding it.
  unsigned epoch_v = __hip_atomic_load(&ctrl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // (straight-line loads throughout the prologue: a load under a branch makes
  // the compiler wait for every load before it at the first use of any)
  int x0_v = a.x0[tid < a.B ? tid : 0];
  constexpr bool CAND = stage_candidates(HEAD, WT, BB);
  constexpr bool NOISE = TEMP && HEAD == kHeadMarkov;  // noise one step ahead in LDS
  // fixed-latent probe (Fig. 13b): the state is never advanced after step 0
  const bool fixed = a.fixed_latent != 0;
  const bool stage = CAND && !fixed;  // stage the exchange's candidate rows for the next latent
  float2* lred = (float2*)(lds + lse_lds_offset(HEAD, WT, BB));  // [kWaves][kMaxB]
  float2* lraw = lred + kWaves * kMaxB;                           // [entries][64]
  int* lcnt = (int*)(lds + kOffLseCnt);
  const int scratch = lds_scratch_bytes(HEAD, WT, BB) + (NOISE ? BB * a.noise_stride * 4 : 0);
  int lds_before = w * a.lds_tiles + min(w, a.lds_extra);  // LDS tiles of the waves before this one
  if (FULL) {
    lds_before = 0;
    for (int u = 0; u < w; ++u) {
      const int nu = cnt > u ? (cnt - u + NW - 1) / NW : 0;
      lds_before += nu - min(nu, a.reg_tiles);
    }
  }
  char* ldsw = lds + scratch + (size_t)lds_before * TB;

  // One-time shard load (Fig. 4 entry cost): register tiles, then LDS tiles.
  // Every register tile is loaded; one that this wave does not own reads the
  // last tile of W instead (its results are dropped: no row of a slot beyond
  // nreg is ever selected or written).
  v4i wr[Gm::RT][Gm::CH];
#pragma unroll
  for (int i = 0; i < Gm::RT; ++i) {
    const int tile = i < nreg ? tb + w + NW * i : a.tiles - 1;
    const v4i* p = (const v4i*)a.Wp + (size_t)tile * Gm::CH * 64 + ro.lane;
#pragma unroll
    for (int c = 0; c < Gm::CH; ++c) wr[i][c] = p[c * 64];
  }
  // vocabulary row of this lane's result in register group gi, and whether it exists
  // (opaque to the compiler, so that values derived from it are recomputed at
  // every step rather than held in registers for the whole walk)
  auto gv = [&](int gi) {
    int v = (tb + w + NW * (gi * Gm::S + ro.cslot)) * kTileRows + ro.n;
    asm volatile("" : "+v"(v));
    return v;
  };
  // (both tests evaluated, without a short circuit: the opaque row cannot be
  // computed speculatively, so `&&` would put each group's test under a branch)
  auto gok = [&](int gi) { return (gi * Gm::S + ro.cslot < nreg) & (gv(gi) < a.V); };
  float gsw[WT == 0 ? Gm::NG : 1];  // row scales of the register groups (int8)
#pragma unroll
  for (int gi = 0; gi < (WT == 0 ? Gm::NG : 1); ++gi)  // rows past the padded scales read 0
    gsw[gi] = WT == 0 ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                       buf_rsrc(a.sw, (uint32_t)a.tiles * kTileRows * 4u),
                                                       4u * (uint32_t)gv(gi), 0, 0))
                      : 0.0f;
  // (the empty asm keeps the uses of the epoch and of the first state, and
  // the waits for them, behind the shard's loads in program order)
  asm volatile("" : "+v"(epoch_v), "+v"(x0_v)::"memory");
  const int row0 = tb * kTileRows;  // first vocabulary row of this workgroup
  float* noise_lds = NOISE ? (float*)(lds + a.noise_off) : nullptr;
  const float* noise = noise_lds;

  // Base logits of the register-resident groups and the first non-register
  // tile are loaded one step ahead, so their memory latency overlaps the
  // previous step's exchange.
  uint16_t bnx[Gm::NG][Gm::NM][Gm::NE];
  // FULL: LDS tiles in slot groups like the register tiles, base logits loaded ahead
  constexpr int NLG = FULL ? (kFullLdsMax + Gm::S - 1) / Gm::S : 1;
  auto lv = [&](int gl) {
    int v = (tb + w + NW * (nreg + gl * Gm::S + ro.cslot)) * kTileRows + ro.n;
    asm volatile("" : "+v"(v));
    return v;
  };
  auto lok = [&](int gl) { return (gl * Gm::S + ro.cslot < nlds) & (lv(gl) < a.V); };
  uint16_t bnl[NLG][Gm::NM][Gm::NE];
  auto fetch_base = [&](int t) {
#pragma unroll
    for (int gi = 0; gi < Gm::NG; ++gi)
#pragma unroll
      for (int m = 0; m < Gm::NM; ++m) load_base<WT, BB>(a, ro, t, m, gv(gi), gok(gi), bnx[gi][m]);
    if (FULL) {
#pragma unroll
      for (int gl = 0; gl < NLG; ++gl)
#pragma unroll
        for (int m = 0; m < Gm::NM; ++m) load_base<WT, BB>(a, ro, t, m, lv(gl), lok(gl), bnl[gl][m]);
    }
  };

  // While the shard is in flight (only the epoch and the first state, loaded
  // before it, are waited for here): the flags, the first state with its
  // check (rows tid < B, all in wave 0, after the flag's reset in program
  // order) and the candidate slots.
  const int par = __builtin_amdgcn_readfirstlane((int)(epoch_v & 1u));
  if (tid == 0) {
    *sflag = 0;
    *lcnt = 0;
  }
  if (tid < a.B) {
    int x = x0_v;
    if (x < 0 || x >= a.V) {
      latch_error(ctrl, 6u);
      *sflag = 1;
      x = 0;
    }
    sx[tid] = x;
  }
  if (CAND) {
    for (int i = tid; i < 64; i += NT) ((int*)(lds + kOffZero))[i] = 0;
    for (int i = tid; i < kGroups * 2; i += NT) ((unsigned long long*)(lds + kOffCand))[i] = 0ull;
    if (tid == 0) *(int*)(lds + kOffDone) = 0;
  }

  for (int i = 0; i < nlds; ++i) {
    const v4i* p = (const v4i*)a.Wp + (size_t)(tb + w + NW * (nreg + i)) * Gm::CH * 64 + ro.lane;
#pragma unroll
    for (int c = 0; c < Gm::CH; ++c) *(v4i*)(ldsw + (size_t)i * TB + c * 1024 + ro.lane * 16) = p[c * 64];
  }
  float racc[BB];
  float cj = 0.0f;
  __syncthreads();
  if (HEAD == kHeadRecurrent) {
    // A[j][k] -> [k/8][j][k%8] (bf16): 16-byte pieces, A is 16-byte aligned
    uint4* At = (uint4*)(lds + kOffAt);
    for (int i = tid; i < kR * kR / 8; i += NT) {
      const int j = i / (kR / 8), kb = i % (kR / 8);
      At[kb * kR + j] = ((const uint4*)a.A)[i];
    }
    float* h = (float*)(lds + kOffH);
    for (int i = tid; i < a.B * kR; i += NT) h[i] = a.h0[i];
    if (tid >= kThreads - kR) cj = a.c[tid - (kThreads - kR)];
  }
  if (NOISE) make_noise(a, noise_lds, 0, row0, cnt * kTileRows, tid, NT);
  // the other parity's lines, for the next walk (nothing reads them in this
  // one); after the LDS tiles, whose loads would otherwise wait for these
  // stores as well
  clear_next_walk<true, NT>(ctrl, par);
  __syncthreads();
  if (*sflag) return;
  fetch_base(0);
  if (HEAD == kHeadRecurrent) {
    recurrent_matvec<BB>(a, tid, lds, racc);
    // every wave has read h_0 before step 0 overwrites it with h_1 (later
    // steps have the end-of-step barrier between the two)
    __syncthreads();
  }
  if (HEAD == kHeadMarkov && CAND && fixed) {
    // the probe's latent, staged once where later steps read staged rows
    if (tid < 32)
      ((int4*)(lds + kOffRows + (tid < 16 ? 0 : kLoOff - 256)))[tid] = ((const int4*)(a.Eq + (size_t)sx[0] * 512))[tid];
    if (tid == 0) {
      ((float*)(lds + kOffShs))[0] = a.Es[sx[0]];
      ((int*)(lds + kOffWin))[0] = 0;
    }
  }

  // One wave per SIMD: the register tiles live in the AGPRs, from which the
  // MFMAs read their B operands directly (without this the compiler keeps
  // them as VGPR values parked in AGPRs and copies each 16-byte chunk back to
  // VGPRs before every use: 4 VALU instructions per MFMA).
  if constexpr (NW == 4) {
    // (the whole-shard variant holds more tiles than the AGPRs: those that fit)
    constexpr int PIN = FULL ? WTS_PIN_FULL : Gm::RT;
#pragma unroll
    for (int i = 0; i < PIN; ++i)
#pragma unroll
      for (int c = 0; c < Gm::CH; ++c) asm volatile("" : "+a"(wr[i][c]));
  }
  // per-step phase stamps (workgroup view of wave 0)
  auto stamp = [&](int t, int k) {
    if (a.trace && tid == 0) a.trace[((size_t)t * G + g) * 4 + k] = wall_clock64();
  };
  for (int t = 0; t < a.gamma; ++t) {
    stamp(t, 0);
    // state -> latent (Markov: embedding row of x_t; recurrent: h_{t+1})
    if (HEAD == kHeadRecurrent && (t == 0 || !fixed))
      recurrent_advance<WT, BB>(a, tid, sx, lds, racc, cj, stage && t > 0);
    // scales of the latent rows (int8), issued with the latent gather
    float shi[Gm::NM][Gm::NE];
#pragma unroll
    for (int m = 0; m < Gm::NM; ++m)
#pragma unroll
      for (int e = 0; e < Gm::NE; ++e) {
        const int b = ro.bent(m, e);
        shi[m][e] = 0.0f;
        if (WT == 0 && b < BB && b < a.B) {
          if (HEAD == kHeadMarkov && CAND && t > 0)
            shi[m][e] = ((const float*)(lds + kOffShs))[((const int*)(lds + kOffWin))[b]];
          else
            shi[m][e] = HEAD == kHeadMarkov ? a.Es[sx[b]] : ((const float*)(lds + kOffShi))[b];
        }
      }
    // first non-register tile of this step: its load overlaps the register tiles' work
    TileBuf<WT, BB> first;
    if (!FULL && nreg < nw) fetch_tile<WT, BB, NW>(a, ro, t, tb, w, nreg, nreg, nlds, ldsw, first);
    v4i lat[Gm::NM][Gm::CH];
    if (HEAD == kHeadMarkov && CAND && t > 0)
      load_latent_staged<WT, BB>(a, ro, lds, lat);
    else
      load_latent<WT, BB, HEAD>(a, ro, sx, lds, lat);
    if (a.trace) {
      __builtin_amdgcn_s_waitcnt(0);
      stamp(t, 1);
    }
    typename LKey<TEMP>::T best[Gm::NM][Gm::NE];
#pragma unroll
    for (int m = 0; m < Gm::NM; ++m)
#pragma unroll
      for (int e = 0; e < Gm::NE; ++e) best[m][e] = 0;
    LseAcc<Gm::NM, Gm::NE, LS> ls;
    ls.init();
    // T=1, three or four rows: the register groups' noise read from LDS now,
    // so that the epilogues do not wait for it (measured slower at one row)
    constexpr bool GP = NOISE && BB == 4;
    float gzp[GP ? Gm::NG : 1][Gm::NM][Gm::NE];
    if constexpr (GP) {
#pragma unroll
      for (int gi = 0; gi < Gm::NG; ++gi)
#pragma unroll
        for (int m = 0; m < Gm::NM; ++m)
#pragma unroll
          for (int e = 0; e < Gm::NE; ++e) {
            const int b = ro.bent(m, e);
            const bool okb = b < BB && gok(gi) && b < a.B;
            gzp[gi][m][e] = noise[okb ? b * a.noise_stride + (gv(gi) - row0) : 0];
          }
    }

    // projection over the register-resident tiles, S tiles per accumulator
#pragma unroll
    for (int gi = 0; gi < Gm::NG; ++gi) {
      // (whole-shard kernels: every group, so that the groups and their
      // epilogues form one block; a slot past the wave's tiles is dropped by gok)
      if (FULL || gi * Gm::S < nreg) {
#pragma unroll
        for (int m = 0; m < Gm::NM; ++m) {
          // One accumulator per tile of the group (independent MFMA chains).
          // A single-tile int8 group splits its chunks over two chains, summed
          // exactly at the end; bf16 keeps one chain per tile (the fp32 order
          // of every execution mode is the same: chunk 0..7 per tile).
          AT accs[Gm::S], acc2 = {0, 0, 0, 0};
          constexpr bool SPLIT = WT == 0 && Gm::S == 1;
#pragma unroll
          for (int s = 0; s < Gm::S; ++s) accs[s] = AT{0, 0, 0, 0};
          // chunk-major over the group's register tiles (independent MFMA
          // chains); a slot past this wave's tiles holds a copy of the last
          // tile of W, whose results are never selected (gok), so the group's
          // tiles are computed without a run-time test
#pragma unroll
          for (int c = 0; c < Gm::CH; ++c)
#pragma unroll
            for (int s = 0; s < Gm::S; ++s) {
              const int i = gi * Gm::S + s;
              if (i < Gm::RT) {  // compile-time: the slots that exist in registers
                if (SPLIT && (c & 1)) acc2 = mma(lat[m][c], wr[i][c], acc2);
                else accs[s] = mma(lat[m][c], wr[i][c], accs[s]);
              }
            }
          AT acc = pick_slot<Gm::S>(accs, ro.cslot);
          if (SPLIT) acc = acc + acc2;
          epilogue<WT, BB, TEMP, NOISE, LS, GP, FULL>(a, ro, t, m, acc, gv(gi), 0xFFFFu - (uint32_t)(gv(gi) - row0),
                                                gok(gi), WT == 0 ? gsw[gi] : 0.0f, bnx[gi][m], shi, best, ls,
                                                noise, row0, gzp[GP ? gi : 0][m]);
        }
      }
    }
    // LDS-resident and streamed tiles
    if (FULL) {
      // LDS tiles only, S per group, their chunks read straight into the MFMA operands,
      // LR reads in flight (as many as the registers left over allow)
      constexpr int LR = BB == 1 ? WTS_LDS_RING_1 : BB == 2 ? WTS_LDS_RING_2 : WTS_LDS_RING_4;
#pragma unroll
      for (int gl = 0; gl < NLG; ++gl) {
        if (gl * Gm::S < nlds) {
          __builtin_amdgcn_sched_barrier(0);  // one group's chunks in flight at a time (registers)
#pragma unroll
          for (int m = 0; m < Gm::NM; ++m) {
            AT accs[Gm::S];
#pragma unroll
            for (int s = 0; s < Gm::S; ++s) accs[s] = AT{0, 0, 0, 0};
            auto lds_chunk = [&](int s, int c) {
              return *(const v4i*)(ldsw + (size_t)(gl * Gm::S + s) * TB + c * 1024 + ro.lane * 16);
            };
            if ((gl + 1) * Gm::S <= nlds) {
              // a full group: chunk-major, no per-MFMA test; the chunk reads run
              // LR ahead of the MFMAs that take them (read, wait, multiply one
              // chunk at a time costs a whole LDS round trip per MFMA)
              constexpr int NJ = Gm::CH * Gm::S;
              v4i ring[LR];
#pragma unroll
              for (int j = 0; j < LR; ++j) ring[j] = lds_chunk(j % Gm::S, j / Gm::S);
#pragma unroll
              for (int j = 0; j < NJ; ++j) {
                accs[j % Gm::S] = mma(lat[m][j / Gm::S], ring[j % LR], accs[j % Gm::S]);
                if (j + LR < NJ) ring[j % LR] = lds_chunk((j + LR) % Gm::S, (j + LR) / Gm::S);
              }
            } else {
              // the last, partial group: one test per tile, its chunks read ahead the same way
#pragma unroll
              for (int s = 0; s < Gm::S; ++s)
                if (gl * Gm::S + s < nlds) {
                  v4i ring[LR];
#pragma unroll
                  for (int c = 0; c < LR; ++c) ring[c] = lds_chunk(s, c);
#pragma unroll
                  for (int c = 0; c < Gm::CH; ++c) {
                    accs[s] = mma(lat[m][c], ring[c % LR], accs[s]);
                    if (c + LR < Gm::CH) ring[c % LR] = lds_chunk(s, c + LR);
                  }
                }
            }
            const int v = lv(gl);
            epilogue<WT, BB, TEMP, NOISE, LS, false, true>(a, ro, t, m, pick_slot<Gm::S>(accs, ro.cslot), v,
                                              0xFFFFu - (uint32_t)(v - row0), lok(gl), 0.0f, bnl[gl][m], shi,
                                              best, ls, noise, row0);
          }
        }
      }
    } else if (nreg < nw) {
      // two tile buffers unless the registers are short (T=1 at sixteen int8 rows, recurrent at T=1);
      // three for sixteen bf16 rows (one wave per SIMD; measured slower at eight rows), except
      // in the greedy walk without log normaliser, whose registers hold a seventh register tile
      // instead (measured faster: fewer tiles stream)
      constexpr int PD = TEMP == 1 && (HEAD == kHeadRecurrent || (WT == 0 && BB >= 16)) ? 1
                         : NW == 4 && BB == 16 && TEMP + (LS ? 1 : 0) == 1               ? 3
                                                                                          : 2;
      stream_tiles<WT, BB, TEMP, NW, NOISE, LS, PD>(a, ro, t, tb, w, nreg, nlds, nw, ldsw, first, lat, shi, best,
                                                    ls, noise);
    }
    if (t + 1 < a.gamma) fetch_base(t + 1);

    // Fig. 8: local winner -> device-scope max key and arrival count -> wait
    // for every workgroup -> common winner.
    reduce_to_lds<WT, BB, TEMP>(ro, w, best, red);
    if (w == 0) lse_stash<WT, BB, LS>(ro, ls, lraw);
    __syncthreads();
    stamp(t, 2);
    // the workgroup's log-sum-exp pairs of this step, merged during the exchange
    if (w > 0) lse_workgroup<WT, BB, NW, LS>(a, ro, w, ls, lred, lraw, lcnt, t, g, G);
    // (no reads of candidate rows during the exchange from two rows on: the
    // exchange's hops slow down under memory traffic by more than the gather
    // after it gains)
    if constexpr (CAND) {
      if (stage && w == 1 && t + 1 < a.gamma) stage_rows<HEAD, BB>(a, t, lds, a.timeout_ticks);
    }
    // next step's base-logit lines into the L2 when some tiles are not in
    // registers (greedy Markov walks; at T=1 these waves make the noise)
    constexpr bool TOUCH = !FULL && !NOISE && HEAD == kHeadMarkov;
    const bool touch = TOUCH && cnt > NW * a.reg_tiles && t + 1 < a.gamma && w >= (CAND ? 2 : 1);
    BaseTouch bt{};
    if (touch) bt = touch_base(a, t + 1, row0, cnt * kTileRows, tid - (CAND ? 2 : 1) * 64, NT - (CAND ? 2 : 1) * 64);
    // next step's noise while wave 0 (and wave 1 when staging) waits on the exchange
    if (NOISE && t + 1 < a.gamma && w >= (CAND ? 2 : 1))
      make_noise(a, noise_lds, t + 1, row0, cnt * kTileRows, tid - (CAND ? 2 : 1) * 64, NT - (CAND ? 2 : 1) * 64);
    if (touch) touch_done(bt, lds + kOffFlag + 4);
    if (w == 0) {
      const int lane = ro.lane;
      unsigned long long k = 0ull;
      if (lane < a.B) {
        typename LKey<TEMP>::T lk = 0;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) lk = kmax(lk, (typename LKey<TEMP>::T)red[ww * kMaxB + lane]);
        k = global_key(lk, row0);
      }
      if (a.stress) {
        // testing aid: arrive late by a pseudo-random 0..15 x 128 cycles
        uint32_t h = (uint32_t)g * 0x9E3779B1u ^ (uint32_t)(t + 1) * 0x85EBCA77u ^ a.seed_lo;
        h ^= h >> 15;
        h *= 0x2C1B3C6Du;
        h ^= h >> 13;
        const int n = __builtin_amdgcn_readfirstlane((int)(h & 15u));
        for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(2);
      }
      unsigned long long win;
      const bool ok = exchange<BB, CAND>(ctrl, par, t, a.B, k, a.timeout_ticks, &win, lds, a.xcd_l1 != 0);
      if (!ok && lane == 0) {
        latch_error(ctrl, 5u);
        *sflag = 1;
      }
      if (lane < a.B) {
        if (a.winners != nullptr) a.winners[(unsigned)((t * a.B + lane) * G + g)] = win;
        int x = key_token(win);
        if (!ok || x < 0 || x >= a.V) {  // only after a failed exchange; keep every access in bounds
          if (ok) latch_error(ctrl, 5u);
          *sflag = 1;
          x = 0;
        }
        if (!fixed) sx[lane] = x;
        if (g == 0) a.tokens[lane * a.gamma + t] = x;
      }
      stamp(t, 3);
    }
    // recurrent: A h_{t+1} for the next step while wave 0 waits
    if (HEAD == kHeadRecurrent && t + 1 < a.gamma && !fixed) recurrent_matvec<BB>(a, tid, lds, racc);
    __syncthreads();
    if (*sflag) return;
  }
  // Workgroup 0 has finished its last exchange, so every workgroup has read
  // the epoch: the next walk may use the other parity.
  if (g == 0 && tid == 0) advance_epoch(ctrl);
  if (HEAD == kHeadRecurrent && g == 0 && a.state) {
    const float* h = (const float*)(lds + kOffH);
    for (int i = tid; i < a.B * kR; i += NT) a.state[i] = h[i];
  }
}

// ----------------------------------------------------------------------------
// step-wise baseline: one launch per step, W streamed every step
// ----------------------------------------------------------------------------

constexpr int kStepWaves = 4;

template <int WT, int BB, int TEMP, bool LS>
__global__ __launch_bounds__(kStepWaves * 64) void step_kernel(WalkArgs a) {
  using Gm = Geo<WT, BB>;
  __shared__ unsigned long long red[kWaves * kMaxB];
  __shared__ float2 lred[LS ? kStepWaves * kMaxB : 1];
  __shared__ int sx[kMaxB];
  const int tid = threadIdx.x, w = tid >> 6;
  const Roles<WT, BB> ro(tid & 63);
  const int g = blockIdx.x, G = gridDim.x;
  const int t = a.step;
  Ctrl* ctrl = a.ctrl;
  const int par = walk_parity(ctrl);
  if (t == 0) clear_next_walk<false>(ctrl, par);
  if (tid < a.B) {
    int x = a.x0[tid];
    if (t > 0) {
      unsigned long long k = 0ull;
#pragma unroll
      for (int i = 0; i < kSub; ++i) k = umax64(k, ld_agent(&ctrl->ss[par][t - 1][tid][i]));
      const int xt = key_token(k);
      if (g == 0) a.tokens[tid * a.gamma + t - 1] = xt;
      if (!a.fixed_latent) x = xt;  // the fixed-latent probe keeps the latent of x0
    }
    if (x < 0 || x >= a.V) {
      latch_error(ctrl, 6u);
      x = 0;
    }
    sx[tid] = x;
  }
  __syncthreads();
  const int tb = (int)((long long)g * a.tiles / G);
  const int te = (int)((long long)(g + 1) * a.tiles / G);
  const int cnt = te - tb;
  const int nw = cnt > w ? (cnt - w + kStepWaves - 1) / kStepWaves : 0;
  float shi[Gm::NM][Gm::NE];
#pragma unroll
  for (int m = 0; m < Gm::NM; ++m)
#pragma unroll
    for (int e = 0; e < Gm::NE; ++e) {
      const int b = ro.bent(m, e);
      shi[m][e] = (WT == 0 && b < BB && b < a.B) ? a.Es[sx[b]] : 0.0f;
    }
  v4i lat[Gm::NM][Gm::CH];
  load_latent<WT, BB, kHeadMarkov>(a, ro, sx, nullptr, lat);
  typename LKey<TEMP>::T best[Gm::NM][Gm::NE];
#pragma unroll
  for (int m = 0; m < Gm::NM; ++m)
#pragma unroll
    for (int e = 0; e < Gm::NE; ++e) best[m][e] = 0;
  LseAcc<Gm::NM, Gm::NE, LS> ls;
  ls.init();
  if (nw > 0) {
    TileBuf<WT, BB> first;
    fetch_tile<WT, BB, kStepWaves>(a, ro, t, tb, w, 0, 0, 0, nullptr, first);
    stream_tiles<WT, BB, TEMP, kStepWaves, false, LS, 2>(a, ro, t, tb, w, 0, 0, nw, nullptr, first, lat, shi,
                                                            best, ls, (const float*)nullptr);
  }
  reduce_to_lds<WT, BB, TEMP>(ro, w, best, red);
  lse_reduce_to_lds<WT, BB, LS>(ro, w, ls, lred);
  __syncthreads();
  if (LS && w == 1) lse_store_partial(a, lred, kStepWaves, t, g, G, ro.lane);
  if (tid < a.B) {
    typename LKey<TEMP>::T lk = 0;
    for (int ww = 0; ww < kStepWaves; ++ww) lk = kmax(lk, (typename LKey<TEMP>::T)red[ww * kMaxB + tid]);
    const unsigned long long k = global_key(lk, tb * kTileRows);
    __hip_atomic_fetch_max(&ctrl->ss[par][t][tid][g % kSub], k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Last token of a step-wise walk; then the walk's epoch advances.
__global__ void finish_kernel(WalkArgs a) {
  const int b = threadIdx.x;
  const int par = walk_parity(a.ctrl);
  if (b < a.B) {
    unsigned long long k = 0ull;
    for (int i = 0; i < kSub; ++i) k = umax64(k, ld_agent(&a.ctrl->ss[par][a.gamma - 1][b][i]));
    const int x = key_token(k);
    a.tokens[b * a.gamma + a.gamma - 1] = (x >= 0 && x < a.V) ? x : 0;
  }
  __syncthreads();
  if (b == 0) advance_epoch(a.ctrl);
}

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------

hipError_t launch_repack_i8(const int8_t* W, const float* w_scale, int V, int tiles, int4* Wp,
                            float* sw, hipStream_t s) {
  const long long total = (long long)tiles * kChunksI8 * 64;
  repack_i8_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(W, w_scale, V, tiles, Wp, sw);
  return hipGetLastError();
}

hipError_t launch_repack_bf16(const uint16_t* W, int V, int tiles, int4* Wp, hipStream_t s) {
  const long long total = (long long)tiles * kChunksBF * 64;
  repack_bf16_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(W, V, tiles, Wp);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const float* E, int V, int8_t* Eq, float* Es, hipStream_t s) {
  quant_rows_kernel<<<(V + 3) / 4, 256, 0, s>>>(E, V, Eq, Es);
  return hipGetLastError();
}

hipError_t launch_bf16_rows(const float* E, int V, uint16_t* Eb, hipStream_t s) {
  const long long n = (long long)V * kR;
  bf16_rows_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(E, n, Eb);
  return hipGetLastError();
}

// The persistent kernel needs all `grid` workgroups resident at once.  With
// grid <= CUs and more than half of a CU's LDS per workgroup, a plain launch
// places one workgroup per CU on an otherwise idle GPU; the cooperative
// launch guarantees it but costs ~18 us more per launch on MI355X.  Either
// way a workgroup that waits too long in the exchange latches WTS_ERR_TIMEOUT
// and exits, so the grid always drains.
template <int WT, int BB, int HEAD, int TEMP, bool LS>
static hipError_t launch_walk_t(const WalkArgs& a, int grid, int lds_bytes, bool coop, hipStream_t s) {
  void* args[] = {(void*)&a};
  const void* fn = (const void*)walk_kernel<WT, BB, HEAD, TEMP, LS, false>;
  if constexpr (reg_tiles_full(HEAD, WT, BB) > 0)
    if (a.full) fn = (const void*)walk_kernel<WT, BB, HEAD, TEMP, LS, true>;
  const dim3 blk(waves_for(HEAD, WT) * 64);
  if (coop) return hipLaunchCooperativeKernel(fn, dim3(grid), blk, args, (unsigned)lds_bytes, s);
  return hipLaunchKernel(fn, dim3(grid), blk, args, (size_t)lds_bytes, s);
}

template <int WT, int HEAD, int TEMP, bool LS>
static hipError_t launch_walk_bb(int BB, const WalkArgs& a, int grid, int lds_bytes, bool coop, hipStream_t s) {
  switch (BB) {
    case 1: return launch_walk_t<WT, 1, HEAD, TEMP, LS>(a, grid, lds_bytes, coop, s);
    case 2: return launch_walk_t<WT, 2, HEAD, TEMP, LS>(a, grid, lds_bytes, coop, s);
    case 4: return launch_walk_t<WT, 4, HEAD, TEMP, LS>(a, grid, lds_bytes, coop, s);
    case 8: return launch_walk_t<WT, 8, HEAD, TEMP, LS>(a, grid, lds_bytes, coop, s);
    case 16: return launch_walk_t<WT, 16, HEAD, TEMP, LS>(a, grid, lds_bytes, coop, s);
  }
  return hipErrorInvalidValue;
}

template <int WT, int HEAD>
static hipError_t launch_walk_temp(int BB, const WalkArgs& a, int grid, int lds_bytes, bool coop, hipStream_t s) {
  if (a.lse)
    return a.temperature ? launch_walk_bb<WT, HEAD, 1, true>(BB, a, grid, lds_bytes, coop, s)
                         : launch_walk_bb<WT, HEAD, 0, true>(BB, a, grid, lds_bytes, coop, s);
  return a.temperature ? launch_walk_bb<WT, HEAD, 1, false>(BB, a, grid, lds_bytes, coop, s)
                       : launch_walk_bb<WT, HEAD, 0, false>(BB, a, grid, lds_bytes, coop, s);
}

hipError_t launch_walk(int wtype, int BB, const WalkArgs& a, int grid, int lds_bytes, bool coop, hipStream_t s) {
  if (wtype == 0)
    return a.head == kHeadMarkov ? launch_walk_temp<0, kHeadMarkov>(BB, a, grid, lds_bytes, coop, s)
                                 : launch_walk_temp<0, kHeadRecurrent>(BB, a, grid, lds_bytes, coop, s);
  return a.head == kHeadMarkov ? launch_walk_temp<1, kHeadMarkov>(BB, a, grid, lds_bytes, coop, s)
                               : launch_walk_temp<1, kHeadRecurrent>(BB, a, grid, lds_bytes, coop, s);
}

template <int WT, int TEMP, bool LS>
static hipError_t launch_step_t(int BB, const WalkArgs& a, int grid, hipStream_t s) {
  const dim3 blk(kStepWaves * 64);
  switch (BB) {
    case 1: step_kernel<WT, 1, TEMP, LS><<<grid, blk, 0, s>>>(a); break;
    case 2: step_kernel<WT, 2, TEMP, LS><<<grid, blk, 0, s>>>(a); break;
    case 4: step_kernel<WT, 4, TEMP, LS><<<grid, blk, 0, s>>>(a); break;
    case 8: step_kernel<WT, 8, TEMP, LS><<<grid, blk, 0, s>>>(a); break;
    case 16: step_kernel<WT, 16, TEMP, LS><<<grid, blk, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int WT>
static hipError_t launch_step_w(int BB, const WalkArgs& a, int grid, hipStream_t s) {
  if (a.lse)
    return a.temperature ? launch_step_t<WT, 1, true>(BB, a, grid, s) : launch_step_t<WT, 0, true>(BB, a, grid, s);
  return a.temperature ? launch_step_t<WT, 1, false>(BB, a, grid, s) : launch_step_t<WT, 0, false>(BB, a, grid, s);
}

hipError_t launch_step(int wtype, int BB, const WalkArgs& a, int grid, hipStream_t s) {
  return wtype == 0 ? launch_step_w<0>(BB, a, grid, s) : launch_step_w<1>(BB, a, grid, s);
}

hipError_t launch_finish(const WalkArgs& a, hipStream_t s) {
  finish_kernel<<<1, 64, 0, s>>>(a);
  return hipGetLastError();
}

// Every reduced log_p argument (one thread per mantissa): counts where
// log_ratio differs from the IEEE quotient.
__global__ __launch_bounds__(256) void check_log_ratio_kernel(unsigned long long* mismatches) {
  const uint32_t k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= (1u << 23)) return;
  float m = __uint_as_float(k | 0x3F000000u);
  if (m < 0.70710677f) m = m * 2.0f;
  const float f = m - 1.0f;
  const float ieee = f / (2.0f + f);
  if (__float_as_uint(log_ratio(f)) != __float_as_uint(ieee)) atomicAdd(mismatches, 1ull);
}

hipError_t launch_check_log_ratio(unsigned long long* mismatches, hipStream_t s) {
  check_log_ratio_kernel<<<(1u << 23) / 256, 256, 0, s>>>(mismatches);
  return hipGetLastError();
}

// XCD (XCC) that workgroup g runs on, from the hardware register XCC_ID
// (bits 3:0), one entry per workgroup.
__global__ void xcc_id_kernel(unsigned* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = (unsigned)__builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 0xFu;
}

hipError_t launch_xcc_ids(unsigned* out, int grid, hipStream_t s) {
  xcc_id_kernel<<<grid, 64, 0, s>>>(out);
  return hipGetLastError();
}

// Zero `bytes` (a multiple of 16) of device memory with a kernel.
__global__ void fill_zero_kernel(int4* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_int4(0, 0, 0, 0);
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 16;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 1024);
  fill_zero_kernel<<<blocks, 256, 0, s>>>((int4*)p, n);
  return hipGetLastError();
}

hipError_t launch_lse(const WalkArgs& a, int grid, hipStream_t s) {
  const int pairs = a.B * a.gamma;
  lse_kernel<<<(pairs + kLseWaves - 1) / kLseWaves, kLseWaves * 64, 0, s>>>(a, grid);
  return hipGetLastError();
}

template <int WT, int HEAD, int TEMP, bool LS>
static hipError_t set_lds_attr(int lds_bytes) {
  hipError_t e = hipSuccess;
  const void* fns[] = {
      (const void*)walk_kernel<WT, 1, HEAD, TEMP, LS, false>, (const void*)walk_kernel<WT, 2, HEAD, TEMP, LS, false>,
      (const void*)walk_kernel<WT, 4, HEAD, TEMP, LS, false>, (const void*)walk_kernel<WT, 8, HEAD, TEMP, LS, false>,
      (const void*)walk_kernel<WT, 16, HEAD, TEMP, LS, false>};
  for (const void* f : fns) {
    const hipError_t r = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (r != hipSuccess) e = r;
  }
  if constexpr (reg_tiles_full(HEAD, WT, 1) > 0) {
    const void* full[] = {(const void*)walk_kernel<WT, 1, HEAD, TEMP, LS, true>,
                          (const void*)walk_kernel<WT, 2, HEAD, TEMP, LS, true>,
                          (const void*)walk_kernel<WT, 4, HEAD, TEMP, LS, true>};
    for (const void* f : full) {
      const hipError_t r = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
      if (r != hipSuccess) e = r;
    }
  }
  return e;
}

template <bool LS>
static hipError_t set_lds_attr_all(int lds_bytes) {
  const hipError_t r[] = {
      set_lds_attr<0, kHeadMarkov, 0, LS>(lds_bytes), set_lds_attr<0, kHeadMarkov, 1, LS>(lds_bytes),
      set_lds_attr<0, kHeadRecurrent, 0, LS>(lds_bytes), set_lds_attr<0, kHeadRecurrent, 1, LS>(lds_bytes),
      set_lds_attr<1, kHeadMarkov, 0, LS>(lds_bytes), set_lds_attr<1, kHeadMarkov, 1, LS>(lds_bytes),
      set_lds_attr<1, kHeadRecurrent, 0, LS>(lds_bytes), set_lds_attr<1, kHeadRecurrent, 1, LS>(lds_bytes)};
  for (hipError_t e : r)
    if (e != hipSuccess) return e;
  return hipSuccess;
}

hipError_t prepare_kernels(int lds_bytes) {
  const hipError_t e = set_lds_attr_all<false>(lds_bytes);
  return e != hipSuccess ? e : set_lds_attr_all<true>(lds_bytes);
}


// ----------------------------------------------------------------------------
// roofline microbenchmarks: the denominators of the walk's rooflines,
// measured on the device the walk runs on (one workgroup per CU where the
// walk has one)
// ----------------------------------------------------------------------------

// Aggregate LDS read rate: every lane reads 16 bytes per ds_read_b128 from
// its own consecutive chunk (no bank conflicts), 8 reads in flight per round;
// the round's offset is made opaque so that no read can leave the loop.
__global__ __launch_bounds__(512) void rf_lds_kernel(int rounds, unsigned* out) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  for (int i = tid; i < 65536 / 16; i += blockDim.x) ((int4*)lds)[i] = make_int4(i, i ^ 1, i ^ 2, i ^ 3);
  __syncthreads();
  v4i acc = {0, 0, 0, 0};
  typedef const __attribute__((address_space(3))) v4i lds_v4i;
  for (int r = 0; r < rounds; ++r) {
    int base = ((r & 7) * 8192 + tid * 16) & 65535;
    asm volatile("" : "+v"(base));
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= *(lds_v4i*)(lds + ((base + u * 8192) & 65535));
  }
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x12345678) out[blockIdx.x] = 1u;
}

// Dense MFMA issue rate: 8 independent accumulator chains per wave with
// register operands.  Thread 0 of each workgroup also records the shader
// clock (s_memtime) and the 100 MHz wall clock at the start and the end.
template <int WT>
__global__ __launch_bounds__(512) void rf_mfma_kernel(int rounds, unsigned* out, long long* clk) {
  using AT = typename AccT<WT>::T;
  const int lane = threadIdx.x & 63;
  v4i a = {lane, lane * 3, lane * 5, lane * 7}, b = {lane * 11, lane * 13, lane ^ 7, lane ^ 9};
  if (WT == 1) {  // small bf16 values (no overflow): bit patterns of numbers near 1
    a = v4i{0x3F803F80, 0x3F813F82, 0x3F833F84, 0x3F853F86};
    b = v4i{0x3F873F88, 0x3F893F8A, 0x3F8B3F8C, 0x3F8D3F8E};
  }
  AT c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = AT{0, 0, 0, 0};
  long long t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = (long long)__builtin_amdgcn_s_memtime();
    r0 = wall_clock64();
  }
  for (int r = 0; r < rounds; ++r) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = mma(a, b, c[i]);
  }
  if (threadIdx.x == 0) {
    const long long t1 = (long long)__builtin_amdgcn_s_memtime(), r1 = wall_clock64();
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += (float)c[i][0] + (float)c[i][3];
  if (s == 1234.5f) out[blockIdx.x] = 1u;
}

// Streaming read of n 16-byte words, `passes` times over (grid-stride,
// coalesced, 8 loads in flight per lane).
__global__ __launch_bounds__(256) void rf_stream_kernel(const int4* __restrict__ p, long long n, int passes,
                                                        unsigned* out) {
  int4 acc = make_int4(0, 0, 0, 0);
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (int pass = 0; pass < passes; ++pass) {
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 7 * stride < n; i += 8 * stride) {
      int4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = p[i + u * stride];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc.x ^= x[u].x;
        acc.y ^= x[u].y;
        acc.z ^= x[u].z;
        acc.w ^= x[u].w;
      }
    }
    for (; i < n; i += stride) {
      const int4 x = p[i];
      acc.x ^= x.x;
      acc.y ^= x.y;
      acc.z ^= x.z;
      acc.w ^= x.w;
    }
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x13572468) out[blockIdx.x] = 1u;
}

// Rounds of one cross-workgroup selection with nothing else in between,
// one wave per workgroup, one workgroup per CU.  variant 0: the walk's
// two-level all-gather with the first level inside an XCD; 1: the same at
// device scope; 2: a flat all-gather (every workgroup stores its key in 8
// per-XCD copies and polls all G keys of its copy); 3: Fig. 8 as drawn, a
// device-scope atomic maximum on one slot and an arrival counter.  Thread 0
// of each workgroup records the wall clock around the rounds; every
// workgroup checks that it saw the true maximum (wrong[g] counts misses,
// timed_out[g] counts expired waits).
__device__ __forceinline__ unsigned long long rf_key(int g, int r) {
  // distinct keys with a step-dependent winner, below the step tag
  const uint32_t h = (uint32_t)(g * 2654435761u) ^ (uint32_t)(r * 40503u);
  return ((unsigned long long)(h & 0xFFFFFu) << 18) | (unsigned long long)(0x3FFFFu - (uint32_t)g);
}

__global__ __launch_bounds__(64) void rf_exchange_kernel(int variant, int rounds, Ctrl* ctrl,
                                                         unsigned long long* flat, unsigned* cnt,
                                                         long long timeout, long long* clk, unsigned* wrong) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x, G = gridDim.x;
  long long r0 = 0;
  if (lane == 0) r0 = wall_clock64();
  unsigned bad = 0, expired = 0;
  for (int r = 0; r < rounds; ++r) {
    const unsigned long long key = rf_key(g, r);
    unsigned long long want_key = 0ull;
    for (int q = lane; q < G; q += 64) want_key = umax64(want_key, rf_key(q, r));
    want_key = umax64(want_key, shfl_xor_u64(want_key, 1));
    want_key = umax64(want_key, shfl_xor_u64(want_key, 2));
    want_key = umax64(want_key, shfl_xor_u64(want_key, 4));
    want_key = umax64(want_key, shfl_xor_u64(want_key, 8));
    want_key = umax64(want_key, shfl_xor_u64(want_key, 16));
    want_key = umax64(want_key, shfl_xor_u64(want_key, 32));
    unsigned long long win = 0ull;
    bool ok = true;
    if (variant <= 1) {
      ok = exchange<1, false>(ctrl, 0, r, 1, key, timeout, &win, lds, variant == 0);
      win = __shfl(win, 0, 64);
    } else if (variant >= 4) {
      ok = exchange<1, false, true>(ctrl, 0, r, 1, key, timeout, &win, lds, variant == 4);
      win = __shfl(win, 0, 64);
    } else if (variant == 2) {
      const unsigned long long tag = (unsigned long long)(r + 1) << kTagShift;
      unsigned long long* F = flat + (size_t)(r & 1) * kCopies * kMaxGrid;
      if (lane < kCopies) st_agent(&F[lane * kMaxGrid + g], tag | key);
      const long long t0 = wall_clock64();
      while (true) {
        bool here = true;
        unsigned long long best = 0ull;
        for (int q = lane; q < G; q += 64) {
          const unsigned long long v = ld_agent(&F[(g % kCopies) * kMaxGrid + q]);
          here = here && (v >> kTagShift) == (unsigned long long)(r + 1);
          best = umax64(best, v & kKeyMask);
        }
        if (__all(here)) {
          best = umax64(best, shfl_xor_u64(best, 1));
          best = umax64(best, shfl_xor_u64(best, 2));
          best = umax64(best, shfl_xor_u64(best, 4));
          best = umax64(best, shfl_xor_u64(best, 8));
          best = umax64(best, shfl_xor_u64(best, 16));
          best = umax64(best, shfl_xor_u64(best, 32));
          win = best;
          break;
        }
        if (wall_clock64() - t0 > timeout) {
          ok = false;
          break;
        }
      }
    } else {
      unsigned long long* slot = flat + r;
      unsigned* c = cnt + r;
      if (lane == 0) {
        __hip_atomic_fetch_max(slot, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        const long long t0 = wall_clock64();
        while (__hip_atomic_load(c, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < (unsigned)G) {
          if (wall_clock64() - t0 > timeout) {
            ok = false;
            break;
          }
        }
        win = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      win = __shfl(win, 0, 64);
      ok = __shfl((int)ok, 0, 64) != 0;
    }
    if (!ok) ++expired;
    else if ((win & kKeyMask) != want_key) ++bad;
    if (!ok) break;
  }
  if (lane == 0) {
    clk[g] = wall_clock64() - r0;
    wrong[2 * g] = bad;
    wrong[2 * g + 1] = expired;
  }
}

// One-way latency between workgroup 0 and workgroup `peer`: they pass a
// counter back and forth `rounds` times.  xcd: plain store and NT poll
// through the shared L2 (both on one XCD); otherwise device scope.
__global__ __launch_bounds__(64) void rf_pingpong_kernel(int peer, int xcd, int rounds, unsigned long long* flag,
                                                         long long timeout, long long* clk) {
  const int g = blockIdx.x;
  if ((g != 0 && g != peer) || threadIdx.x != 0) return;
  const bool first = g == 0;
  const long long r0 = wall_clock64();
  unsigned long long* mine = flag + (first ? 0 : 16);
  const unsigned long long* other = flag + (first ? 16 : 0);
  long long t0 = r0;
  bool ok = true;
  for (int r = 0; r < rounds && ok; ++r) {
    if (first) {
      if (xcd) st_xcd(mine, (unsigned long long)r + 1); else st_agent(mine, (unsigned long long)r + 1);
    }
    while (true) {
      unsigned long long v;
      if (xcd) {
        const unsigned long long* pp[1] = {other};
        unsigned long long vv[1];
        ld_xcd<1>(pp, vv);
        v = vv[0];
      } else {
        v = ld_agent(other);
      }
      if (v == (unsigned long long)r + 1) break;
      if (wall_clock64() - t0 > timeout) {
        ok = false;
        break;
      }
    }
    if (!first) {
      if (xcd) st_xcd(mine, (unsigned long long)r + 1); else st_agent(mine, (unsigned long long)r + 1);
    }
    t0 = wall_clock64();
  }
  clk[first ? 0 : 1] = ok ? wall_clock64() - r0 : -1;
}

// VALU issue: n dependent v_add_f32 per lane (one chain), or the same number
// spread over four independent chains; s_memtime cycles per instruction, one
// entry per wave (waves w and w + 4 of a workgroup share a SIMD).
template <int MODE>
__global__ __launch_bounds__(1024) void rf_valu_kernel(int n, float seed, float* out, long long* clk) {
  // MODE 0: one dependent chain of v_add_f32; 1: four independent chains;
  // 2: four independent chains of v_dot4_i32_i8 (the int8 dot product a
  // VALU projection would use)
  float a0 = seed + threadIdx.x, a1 = a0 * 0.5f, a2 = a0 * 0.25f, a3 = a0 * 0.125f;
  const float d = seed * 1e-7f;
  int i0 = (int)threadIdx.x, i1 = i0 ^ 5, i2 = i0 ^ 9, i3 = i0 ^ 17;
  const int x = (int)(seed * 3.0f) | 0x01010101, y = x ^ 0x00FF00FF;
  const long long t0 = (long long)__builtin_amdgcn_s_memtime();
  for (int i = 0; i < n; i += 16) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (MODE == 0) {
        a0 = a0 + d;
        a0 = a0 + d;
        a0 = a0 + d;
        a0 = a0 + d;
      } else if (MODE == 1) {
        a0 = a0 + d;
        a1 = a1 + d;
        a2 = a2 + d;
        a3 = a3 + d;
      } else {
        i0 = __builtin_amdgcn_sdot4(x, y, i0, false);
        i1 = __builtin_amdgcn_sdot4(x, y, i1, false);
        i2 = __builtin_amdgcn_sdot4(x, y, i2, false);
        i3 = __builtin_amdgcn_sdot4(x, y, i3, false);
      }
      asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(i0), "+v"(i1), "+v"(i2), "+v"(i3));
    }
  }
  const long long t1 = (long long)__builtin_amdgcn_s_memtime();
  if ((threadIdx.x & 63) == 0) clk[threadIdx.x >> 6] = t1 - t0;
  out[threadIdx.x] = a0 + a1 + a2 + a3 + (float)(i0 ^ i1 ^ i2 ^ i3);
}

hipError_t launch_rf_lds(int grid, int rounds, unsigned* out, hipStream_t s) {
  const hipError_t e = hipFuncSetAttribute((const void*)rf_lds_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           96 * 1024);
  if (e != hipSuccess) return e;
  rf_lds_kernel<<<grid, 512, 96 * 1024, s>>>(rounds, out);
  return hipGetLastError();
}
hipError_t launch_rf_mfma(int wtype, int grid, int rounds, unsigned* out, long long* clk, hipStream_t s) {
  if (wtype == 0) rf_mfma_kernel<0><<<grid, 512, 0, s>>>(rounds, out, clk);
  else rf_mfma_kernel<1><<<grid, 512, 0, s>>>(rounds, out, clk);
  return hipGetLastError();
}
hipError_t launch_rf_stream(const void* p, long long n16, int passes, int grid, unsigned* out, hipStream_t s) {
  rf_stream_kernel<<<grid, 256, 0, s>>>((const int4*)p, n16, passes, out);
  return hipGetLastError();
}
hipError_t launch_rf_exchange(int variant, int grid, int rounds, Ctrl* ctrl, unsigned long long* flat, unsigned* cnt,
                              long long timeout, long long* clk, unsigned* wrong, hipStream_t s) {
  const hipError_t e = hipFuncSetAttribute((const void*)rf_exchange_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
  if (e != hipSuccess) return e;
  // more than half the LDS per workgroup: one workgroup per CU, as in the walk
  rf_exchange_kernel<<<grid, 64, 96 * 1024, s>>>(variant, rounds, ctrl, flat, cnt, timeout, clk, wrong);
  return hipGetLastError();
}
hipError_t launch_rf_pingpong(int grid, int peer, int xcd, int rounds, unsigned long long* flag, long long timeout,
                              long long* clk, hipStream_t s) {
  rf_pingpong_kernel<<<grid, 64, 0, s>>>(peer, xcd, rounds, flag, timeout, clk);
  return hipGetLastError();
}
hipError_t launch_rf_valu(int mode, int waves, int n, float* out, long long* clk, hipStream_t s) {
  if (mode == 0) rf_valu_kernel<0><<<1, 64 * waves, 0, s>>>(n, 1.5f, out, clk);
  else if (mode == 1) rf_valu_kernel<1><<<1, 64 * waves, 0, s>>>(n, 1.5f, out, clk);
  else rf_valu_kernel<2><<<1, 64 * waves, 0, s>>>(n, 1.5f, out, clk);
  return hipGetLastError();
}

}  // namespace wts
