/*
 * wts.h -- C ABI of the walk-resident serial draft head library (gfx950).
 *
 * The operation: "Weights That Stay: On-Chip Megakernels for Serial Heads in
 * Speculative Decoding" (arXiv 2611.00506).  A serial draft head walks gamma
 * steps; each step projects a rank-r state through the same immutable V x r
 * vocabulary matrix W, adds base logits, selects one token over the whole
 * vocabulary and advances the state (abstract; Fig. 2).  The library runs
 * the whole walk in one persistent kernel that keeps each compute unit's
 * shard of W on chip (Fig. 1), selects tokens on the GPU across workgroups
 * (Fig. 8) and advances the state in the kernel; it also runs the same walk
 * one launch per step, streaming W every step, for comparison (Fig. 4,
 * Fig. 11).
 *
 * Conventions for every entry point:
 *   - "device pointer" = memory of the GPU selected by `device` (e.g. a torch
 *     tensor's data_ptr()).  The library never frees caller memory.
 *   - Every call returns a wts_status and never aborts or throws.  Errors the
 *     host can see are returned before anything is enqueued; outputs are then
 *     untouched.  Errors only the device can see (x0 out of range, barrier
 *     watchdog) are latched in the context and read with wts_get_error().
 *   - Calls on one context must not overlap (one walk in flight per context
 *     on one stream at a time; use one context per concurrent stream).
 */
#ifndef WTS_H_
#define WTS_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum wts_status {
  WTS_OK = 0,
  WTS_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, size out of range      */
  WTS_ERR_UNSUPPORTED = 2,   /* valid but not built (e.g. r != 256)             */
  WTS_ERR_NO_MEMORY = 3,     /* device allocation failed                        */
  WTS_ERR_DEVICE = 4,        /* HIP runtime / launch / cooperative-launch error */
  WTS_ERR_TIMEOUT = 5,       /* device watchdog expired in the grid barrier     */
  WTS_ERR_TOKEN_RANGE = 6    /* an x0 entry was outside [0, V)                  */
} wts_status;

/* Head kinds (Fig. 13): Markov u_t = E[x_{t-1}];
 * recurrent h_t = tanh(A h_{t-1} + E[x_{t-1}] + c). */
enum { WTS_HEAD_MARKOV = 0, WTS_HEAD_RECURRENT = 1 };

/* Storage of W (Fig. 1: int8 with per-row scales, or bf16). */
enum { WTS_W_INT8 = 0, WTS_W_BF16 = 1 };

/* Execution of a walk.
 *  RESIDENT: one persistent launch; each workgroup keeps its W shard on chip
 *            (registers, then LDS) and streams only what does not fit.
 *  STREAM:   one persistent launch that re-reads every W tile from memory at
 *            every step (whole-walk fusion without residency, Fig. 4/11).
 *  STEPWISE: one launch per step, W streamed every step; the kernel boundary
 *            replaces the grid barrier.
 * All three compute identical tokens and logits. */
enum { WTS_EXEC_RESIDENT = 0, WTS_EXEC_STREAM = 1, WTS_EXEC_STEPWISE = 2 };

/* Walk flags.
 *  FIXED_LATENT: the fixed-latent probe of Fig. 13b.  Every step projects and
 *            selects with the latent of step 0 (Markov: E[x0]; recurrent:
 *            h_1); each step's choice is written to tokens_out but does not
 *            feed back.  It times a step without its state advance.
 *  STRESS:   persistent executions only: before each step's cross-workgroup
 *            selection every workgroup waits a pseudo-random time (0 to about
 *            1 us, from its index, the step and the seed), so that keys arrive
 *            in orders a normal walk rarely produces.  Results are unchanged;
 *            for testing the selection (Fig. 8). */
enum { WTS_WALK_FIXED_LATENT = 1, WTS_WALK_STRESS = 2 };

typedef struct wts_ctx wts_ctx;

typedef struct wts_create_params {
  int32_t V;              /* vocabulary rows, 1 <= V <= 262143                 */
  int32_t r;              /* rank; only 256 is built                           */
  int32_t head;           /* WTS_HEAD_*                                        */
  int32_t wtype;          /* WTS_W_*                                           */
  const void* W;          /* device, [V][r] row-major: int8, or bf16 bits;
                             W, E and A 16-byte aligned                       */
  const float* w_scale;   /* device, [V] fp32 per-row scale (int8 only)        */
  const float* E;         /* device, [V][r] fp32 embedding rows                */
  const uint16_t* A;      /* device, [r][r] bf16 bits (recurrent only)         */
  const float* c;         /* device, [r] fp32 (recurrent only)                 */
  int32_t max_batch;      /* 1..16                                             */
  int32_t max_steps;      /* 1..64                                             */
  int32_t resident_tiles; /* -1: planner's choice.  Otherwise the number of
                             16-row tiles each wave keeps in registers (0..the
                             built maximum); the rest is streamed.            */
  int32_t lds_tiles;      /* -1: planner's choice.  Otherwise 16-row tiles per
                             wave kept in LDS (after the register tiles).     */
  int32_t device;         /* HIP device ordinal                                */
  int32_t cooperative;    /* 0: plain launch of the persistent kernel (one
                             workgroup per CU on an idle GPU; if another kernel
                             holds CUs the walk fails with WTS_ERR_TIMEOUT
                             instead of hanging).  1: cooperative launch, which
                             guarantees co-residency at ~18 us more per walk. */
  int32_t watchdog_us;    /* 0: 2 s.  Otherwise the wall-clock limit, in
                             microseconds (>= 1), of every wait inside a walk;
                             a wait that exceeds it latches WTS_ERR_TIMEOUT and
                             its workgroup exits.                              */
  int32_t grid;           /* 0: one workgroup per compute unit (at most 256).
                             Otherwise that many workgroups (1..256, at most
                             the compute units), each with a larger shard.   */
  int32_t exchange;       /* Cross-workgroup selection (Fig. 8).  0: the first
                             level (16 groups) runs through one XCD's L2 when
                             a create-time check finds workgroup g dispatched
                             to the same XCD as g mod 16, else device scope.
                             1: device scope at both levels.                   */
} wts_create_params;

typedef struct wts_walk_params {
  int32_t B;              /* batch rows, 1..max_batch                          */
  int32_t gamma;          /* steps, 1..max_steps                               */
  int32_t step_offset;    /* step index of t=0 in the noise key (resume)       */
  int32_t temperature;    /* 0 greedy, 1 Gumbel-max; anything else invalid    */
  uint64_t seed;          /* noise key (T=1)                                   */
  const uint16_t* base;   /* device, [B][gamma][V] bf16 bits                   */
  const int32_t* x0;      /* device, [B] tokens before step 0                  */
  const float* h0;        /* device, [B][r] fp32 initial state (recurrent)     */
  int32_t* tokens_out;    /* device, [B][gamma] int32 (required)               */
  uint16_t* logits_out;   /* device, [B][gamma][V] bf16 bits, or NULL          */
  float* state_out;       /* device, [B][r] fp32 final state, or NULL          */
  int32_t exec;           /* WTS_EXEC_*                                        */
  int32_t flags;          /* 0 or WTS_WALK_FIXED_LATENT; other bits invalid    */
  void* stream;           /* hipStream_t (NULL = default stream)               */
  int64_t* trace_out;     /* device, [gamma][grid][4] int64, or NULL.  Persistent
                             executions only: per step and workgroup, wall-clock
                             stamps (100 MHz ticks) at step start, latent
                             loaded, local winner ready, common winner known.
                             Per-step breakdown in the manner of Fig. 13b.     */
  float* lse_out;         /* device, [B][gamma] fp32, or NULL: per step, the
                             log normaliser ln sum_v exp(l_v) of that step's
                             bf16 logits l.  A T=1 walk samples its token from
                             q(v) = exp(l_v - lse) (Gumbel-max, Fig. 10), so
                             log q of the drafted token is l[x_t] - lse: what a
                             lossless verifier needs, without a second pass
                             over the logits.  Accumulated in fp32 in the
                             kernel (online max and rescaled sum).            */
  uint64_t* winners_out;  /* device, [gamma][B][grid] uint64, or NULL.
                             Persistent executions only: the winning selection
                             key each workgroup observed at each step for each
                             batch row (bits 49..18 the score's order code,
                             bits 17..0 0x3FFFF - token).  Every workgroup must
                             observe the same key: a race check of Fig. 8.
                             With WTS_EXEC_STEPWISE (or the STRESS flag there)
                             the walk returns WTS_ERR_UNSUPPORTED.             */
} wts_walk_params;

typedef struct wts_plan {
  int32_t grid;            /* workgroups of the persistent kernel (= CUs)      */
  int32_t waves;           /* waves per workgroup                              */
  int32_t tiles;           /* 16-row tiles of W (ceil(V/16))                   */
  int32_t tiles_per_wave;  /* most tiles any wave owns                         */
  int32_t reg_tiles;       /* per wave, held in registers                      */
  int32_t lds_tiles;       /* per wave, held in LDS                            */
  int32_t stream_tiles;    /* per wave (max), streamed each step               */
  int64_t resident_bytes;  /* W bytes on chip over the whole GPU               */
  int64_t streamed_bytes;  /* W bytes read from memory per step                */
  int64_t w_bytes;         /* V * r * element size                             */
  int32_t exchange;        /* 0: first selection level inside an XCD's L2;
                              1: device scope (see wts_create_params.exchange)  */
} wts_plan;

/* Create a head: validates, plans residency, and copies W into a tile-major
 * layout owned by the context (plus the quantised embedding rows, Fig. 7).
 * Borrows E, A, c: keep them alive until wts_destroy.  Synchronous.
 * WTS_ERR_UNSUPPORTED if a workgroup would own more than 65,535 vocabulary
 * rows (V / grid; the local selection key holds a 16-bit row). */
wts_status wts_create(const wts_create_params* p, wts_ctx** out);

/* Enqueue one walk on p->stream: gamma serial draft steps of the head
 * (Fig. 2), each a projection of the latent against W, the epilogue of
 * Fig. 7, a selection across all workgroups (Fig. 8) and the state advance,
 * with the shard of W kept on chip for the whole walk (Fig. 1; or streamed,
 * Fig. 4/11, per exec).  Asynchronous; inputs must stay alive and
 * unmodified until the stream reaches the walk's end.  Writes tokens_out
 * [b][t] = token chosen at step t, and optionally logits_out and state_out.
 * The walk keeps no host-side state between calls (the control block's
 * parity advances on the device), so a walk captured in a HIP graph may be
 * replayed; the captured pointers' contents may change between replays.
 * WTS_ERR_UNSUPPORTED (before any launch) if the LDS a T=1 Markov walk needs
 * for one step of Gumbel noise (4 bytes per batch row and vocabulary row of a
 * workgroup) does not fit beside the kernel's other LDS data. */
wts_status wts_walk(wts_ctx* ctx, const wts_walk_params* p);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * walk as wts_walk, with the same arguments, outputs and bits, but the
 * scratch its kernels use -- the control block of the cross-workgroup
 * exchange and the step-wise slots, the error word, and the per-workgroup
 * log-normaliser partials -- lives in a fixed array of the library on each
 * GPU (set up and cleared by the first wts_create on that GPU, held until the
 * process ends) instead of in the context.  Allocates nothing and calls no
 * allocating routine.  Limit: the partials of one walk that asks for lse_out
 * must fit in WTS_NOALLOC_LSE_BYTES (8 bytes per batch row, step and
 * workgroup; B * gamma * 256 * 8 for persistent walks on 256 compute units,
 * B * gamma * ceil(V/128) * 8 for step-wise walks); beyond it the call
 * returns WTS_ERR_UNSUPPORTED before anything is enqueued.  Every context on
 * one GPU shares that GPU's array: calls that overlap on one GPU (from any
 * context) race and must not be issued; the array keeps the last walk's
 * contents, and each walk clears what the next one needs at zero.  Device
 * errors of these walks are reported by wts_get_error on any context of that
 * GPU. */
#define WTS_NOALLOC_LSE_BYTES (1 << 20)
wts_status wts_walk_noalloc(wts_ctx* ctx, const wts_walk_params* p);

/* Synchronizes the device, then frees everything the context owns (the
 * repacked W that each walk loads on chip, Fig. 1, the quantised embedding
 * rows and the control block of the selection, Fig. 8).  NULL is ignored. */
void wts_destroy(wts_ctx* ctx);

/* Synchronizes the device and returns the error latched by walks since the
 * last clear (WTS_OK if none).  clear != 0 resets the latch. */
wts_status wts_get_error(wts_ctx* ctx, int clear);

/* Residency (registers, LDS, streamed; Fig. 12 placement, Fig. 10 and 14
 * partial residency) a walk of B batch rows under `exec` and `temperature` uses, when
 * it asks for no lse_out (B selects the batch bucket 1, 2, 4, 8 or 16; larger
 * buckets keep fewer tiles in registers; T=1 Markov walks keep the next step's
 * noise in LDS, which can leave room for fewer LDS tiles).  A Markov walk
 * that asks for lse_out, or runs at T=1, holds one register tile per wave
 * fewer than a greedy one without it at two to eight int8 rows and at four,
 * eight or sixteen bf16 rows. */
wts_status wts_get_plan(const wts_ctx* ctx, int32_t B, int32_t exec, int32_t temperature, wts_plan* out);

/* Static description of a status code. */
const char* wts_status_string(wts_status s);

/* Self-check of a numerical shortcut in the kernels.  A T=1 walk draws
 * Gumbel noise -log(-log U) (Gumbel-max, Fig. 10) with a portable binary32
 * log, which divides f by 2 + f for a reduced argument f = m - 1, m in
 * [sqrt(1/2), sqrt(2)).  The kernels form that quotient from a reciprocal
 * estimate and one fused-multiply-add correction instead of the general
 * IEEE division.  This runs both on `device` for all 2^23 reduced mantissas
 * and writes to *mismatches how many differ (0: the shortcut is the correctly
 * rounded quotient everywhere the log can use it).  Allocates and frees 8
 * bytes of device memory; synchronous.  WTS_ERR_INVALID_ARG for a NULL
 * pointer or a negative device, WTS_ERR_DEVICE on a HIP error. */
wts_status wts_check_log_ratio(int32_t device, int64_t* mismatches);

#ifdef __cplusplus
}
#endif

#endif /* WTS_H_ */
