// gg_kernels.hip -- persistent grouped-GEMM kernels for gfx950 (CDNA4).
//
// One kernel template serves every pass of the grouped GEMM (include/gg.h
// states the operations and the passages that define them).  Each pass is
// the same tile engine fed by a different operand description:
//
//   pass           out tile rows x cols   reduction    A operand          B operand
//   forward        expert rows x n        k            X    (red-contig)  W[g] (red-strided)
//   dgrad          expert rows x k        n            dY   (red-contig)  W[g] (red-contig)
//   wgrad          k x n                  expert rows  X    (red-strided) dY   (red-strided)
//   masked fwd     active rows x n        k            X[e] (red-contig)  W[e] (red-strided)
//   masked dgrad   active rows x k        n            dY[e](red-contig)  W[e] (red-contig)
//   masked wgrad   k x n                  active rows  X[e] (red-strided) dY[e](red-strided)
//   SiLU fwd       as forward, 128 activation columns from a gate/up panel
//   fp8 fwd        expert rows x n        k            X e4m3 (contig)    W[g] [n, k] e4m3 (contig)
//
// (The [E, N, K] weight layout of the bf16 passes is these modes with the
// dimensions exchanged; the host entry points do the mapping.)  Epilogues:
// fp32 straight from the accumulators, or through LDS for bf16, for fp32
// wgrad on short experts, for alpha * P + beta * C, for the grouped bias
// s[i] * bias[g], and for the SiLU-mul activation.
//
// "red-contig" means the reduction index is the contiguous one in memory;
// "red-strided" means the tile's row index is.
//
// Data path (no register staging): every operand tile goes from global
// memory straight into LDS with buffer loads in LDS mode (16 bytes per lane,
// 1 KB per wave instruction), one 64-byte-deep reduction stage at a time
// (32 bf16 or 64 e4m3 values), through a ring of 4 LDS slots, each load
// issued 3 to 6 ping-pong steps before its first reader.  In the row passes the A
// operand is staged two stages at a time instead, so that its loads read
// whole cache lines (the pair layout, stated with dma_pair).  Each operand
// keeps its memory layout in LDS:
//   red-contig  : 256 tile rows x 64 bytes (32 reduction values), the
//                 16-byte chunk c of row r at position c ^ ((r / 4) mod 4);
//                 MFMA fragments come from ds_read_b128.
//   red-strided : 4 blocks of 64 tile rows; in a block, reduction row q holds
//                 the block's 64 values (128 bytes), chunk c of reduction row
//                 q at position c ^ (4 ((q / 2) mod 2)); fragments come from
//                 the transposing LDS read (ds_read_b64_tr_b16), two per
//                 fragment.  Within a group of 16 lanes it hands lane j
//                 element j mod 4 of source lane 4 e + j / 4 as its element e,
//                 so source lanes pointing at 4 values of 4 consecutive
//                 reduction rows deliver 4 consecutive reduction values of one
//                 tile row to each lane -- the MFMA operand layout.
// Both layouts make the fragment reads conflict-free on the 64-bank LDS.
// Ragged edges cost nothing extra: each load's buffer resource ends exactly
// at the last byte the tile may read, and out-of-range loads write zeros into
// LDS, so rows past an expert's end and reduction rows past its length are
// zero (no pad copy; TileOPs issue #1566, "Summary" and "Proposed change").
//
// Work decomposition (no host sync, no workspace): one workgroup per compute
// unit.  Each workgroup decodes the device-side end offsets (or masked_m)
// into LDS -- clamped ends by a prefix max, then a prefix sum of per-expert
// tile counts (wgrad: its experts ranked longest first) -- and walks tiles
// t = blockIdx.x, blockIdx.x + gridDim.x, ...
// Stores are predicated by the buffer range check and per column group, so
// rows that belong to no expert are never written and there is no output
// memset; an expert with no rows costs nothing in forward/dgrad and still
// writes its all-zero dW[g] in wgrad.
//
// MFMA: v_mfma_f32_32x32x16_bf16, fp32 accumulation.  A workgroup is 8 waves
// (2 x 4) over a 256 x 256 output tile; each wave owns 128 x 64, i.e. 4 x 2
// MFMA blocks of 32 x 32 (128 accumulator registers per lane), so two waves
// share each SIMD.  Those two take turns (the ping-pong loops): one issues a
// stage's MFMAs back to back from fragments already in its registers while
// the other reads its next fragments from LDS and issues its share of the
// global->LDS loads, so a load that cannot issue yet or an LDS read in flight
// holds up only the wave that is not computing.  The fp8 forward runs the
// same schedule with v_mfma_scale_f32_32x32x64_f8f6f4 (mainloop8_pp).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gg_internal.h"

namespace gg {

constexpr int BM = 256;          // tile rows
constexpr int BN = 256;          // tile cols
constexpr int BK = 32;           // reduction stage
constexpr int NWAVE = 8;         // waves per workgroup, 2 x 4 over the tile
constexpr int NT = 64 * NWAVE;   // threads per workgroup
constexpr int TM = 4;            // 32-row MFMA blocks per wave (wave tile 128 rows)
constexpr int TN = 2;            // 32-col MFMA blocks per wave (wave tile 64 cols)
constexpr int NSTAGE = 4;        // LDS stages (loads run NSTAGE - 1 stages ahead)
constexpr int OP_BYTES = 256 * BK * 2;      // one operand's stage tile: 16 KB
constexpr int STAGE_BYTES = 2 * OP_BYTES;   // A then B: 32 KB

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

enum Mode {
  FWD = 0, DGRAD = 1, WGRAD = 2, MASKED = 3, MASKED_DGRAD = 4, MASKED_WGRAD = 5,
  FWD_SILU = 6, MASKED_SILU = 7, FP8 = 8, FP8_MASKED = 9
};

// The masked modes are the ragged passes on the masked layout: expert e's
// rows start at e * max_m and its active count is masked_m[e].  The SiLU
// modes are forwards whose epilogue applies the gate/up activation.
constexpr bool is_masked(int mode) {
  return mode == MASKED || mode == MASKED_DGRAD || mode == MASKED_WGRAD || mode == MASKED_SILU ||
         mode == FP8_MASKED;
}
// The fp8 modes: e4m3 operands, X [rows, K] and W [E, N, K] (both
// reduction-contiguous), one power-of-two scale per 128 reduction values.
constexpr bool is_fp8(int mode) { return mode == FP8 || mode == FP8_MASKED; }
constexpr bool is_silu(int mode) { return mode == FWD_SILU || mode == MASKED_SILU; }
constexpr bool is_wgrad(int mode) { return mode == WGRAD || mode == MASKED_WGRAD; }
constexpr bool is_dgrad(int mode) { return mode == DGRAD || mode == MASKED_DGRAD; }

struct Params {
  const uint16_t* a;        // forward/masked/wgrad: X;  dgrad: dY
  const uint16_t* b;        // forward/masked/dgrad: W;  wgrad: dY
  const int32_t* groups;    // end offsets, or masked_m
  void* c;                  // output
  int64_t m;                // rows of X (ragged) or max_m (masked)
  int64_t k;
  int64_t n;
  int32_t num_groups;
  float alpha;              // out = alpha * product + beta * out
  float beta;               // (the output is not read when beta == 0)
  const uint8_t* sa;        // fp8: X's scales, packed (E8M0 bytes, see the fp8 section)
  const uint8_t* sb;        // fp8: W's scales, packed
  const uint16_t* bias;     // row passes: bf16 [E, output cols] added to each row, or null
  const float* bias_scale;  // its per-row factor (absolute row index), or null for 1
};

// Passes whose epilogue can add the grouped bias: the forward, ragged and
// masked.
constexpr bool has_bias(int mode) { return mode == FWD || mode == MASKED; }

// One operand tile: element (tile row r, reduction index q) of the tile
// lives at byte origin + 2 (r * ld + q) (red-contig) or origin + 2 (q * ld +
// r) (red-strided).
struct Operand {
  const uint8_t* origin;
  uint32_t ld_bytes;  // 2 * ld
  int32_t rows;       // red-contig: valid tile rows (>= 1)
  int32_t red;        // valid reduction length
  uint32_t row_tail;  // red-strided: bytes from the tile's first row to the end of a memory row
  uint32_t split;     // red-strided: extra byte offset of tile rows 128.. (the up half of a
                      // gate/up panel; 0 otherwise)
};

constexpr uint32_t kRsrcWord3 = 0x00020000u;   // gfx9 raw buffer, 32-bit dwords
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset every record count here is below

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, (int)kRsrcWord3);
}

// Values every lane of the wave holds alike (decoded from LDS) moved to
// scalar registers, so buffer resources built from them stay scalar.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Opaque copies: the compiler must recompute whatever depends on them where
// they are used, instead of hoisting per-lane constants out of the tile loop
// (which would keep dozens of them live across the main loop).
__device__ __forceinline__ uint32_t opaque_v(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ uint32_t opaque_s(uint32_t v) {
  asm volatile("" : "+s"(v));
  return v;
}

// Stage barrier: this wave's global->LDS loads and LDS operations are
// complete, then all waves meet.  The wait is the builtin (so the compiler
// knows nothing is outstanding afterwards); the barrier is an asm statement
// with a memory clobber so no LDS access moves across it.
constexpr int kWaitVmLgkm0 = 0x0070;   // s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(0)
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
  asm volatile("s_barrier" ::: "memory");
}

// ---- global -> LDS, one stage of one operand ------------------------------------

// A stage tile of one operand is 16 KB of LDS, written by the 4 waves of
// one group with 4 direct-to-LDS loads each: load jj of the group's wave w
// (0..3) fills bytes [4096 w + 1024 jj, +1024), lane i writing 16 bytes at
// 16 i.  Offsets beyond the record count read as zero.
struct DmaCtx {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t voff;      // lane offset of load 0
  uint32_t step;      // extra byte offset per load (scalar offset)
};

// ---- LDS -> MFMA fragments ------------------------------------------------------

// A fragment: 8 consecutive reduction values (sub-step ks, half l / 32) of
// row 32 i + l % 32 of the wave's slice of an operand tile (128 rows of A,
// 64 rows of B).
struct Frags {
  bf16x8 a[TM];
  bf16x8 b[TN];
};

// Lane-dependent part of the fragment addresses of one operand whose wave
// slice starts at tile row r0 (a multiple of 64).  Red-contig: the byte
// offset of chunk 2 ks + l / 32 of row r0 + l % 32, for ks = 0, 1 (the XOR
// swizzle mixes ks with the lane bits).  Red-strided: the offset of the
// 4-value group a source lane points at, for fragment parity i mod 2
// (sub-step, fragment pair and read half are added as immediates).
struct FragAddr {
  uint32_t o[2];
};

template <bool STRIDED>
__device__ __forceinline__ FragAddr frag_addr(int r0, int lane) {
  FragAddr f;
  if constexpr (STRIDED) {
    const int g = lane >> 4, s = lane & 15;
    const int qrow = 8 * (g >> 1) + (s >> 2);                     // reduction row within the sub-step
    const int sw = 4 * ((s >> 3) & 1);                            // (qrow / 2) mod 2 == (s / 8) mod 2
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int chunk = (4 * par + 2 * (g & 1) + ((s & 3) >> 1)) ^ sw;
      f.o[par] = (uint32_t)((r0 / 64) * 4096 + qrow * 128 + 16 * chunk + 8 * (s & 1));
    }
  } else {
    const int row = r0 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int chunk = (2 * ks + (lane >> 5)) ^ ((row >> 2) & 3);
      f.o[ks] = (uint32_t)(row * 64 + 16 * chunk);
    }
  }
  return f;
}

__device__ __forceinline__ bf16x8 read_tr_pair(const uint8_t* lds, uint32_t off) {
  typedef __attribute__((address_space(3))) shortx4 lds_s4;
  const __attribute__((address_space(3))) uint8_t* base = (const __attribute__((address_space(3))) uint8_t*)lds;
  shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(base + off));
  shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(base + off + 4 * 128));
  typedef short shortx8 __attribute__((ext_vector_type(8)));
  shortx8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Fragment i of sub-step ks of one operand.
template <bool STRIDED>
__device__ __forceinline__ bf16x8 read_frag(const uint8_t* lds, const FragAddr& fa, int ks, int i) {
  if constexpr (STRIDED) {
    // block r0 / 64 + i / 2, reduction rows 16 ks + ..., fragment parity i mod 2
    return read_tr_pair(lds, fa.o[i & 1] + (uint32_t)((i >> 1) * 4096 + ks * 16 * 128));
  } else {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(lds + fa.o[ks] + (uint32_t)(i * 32 * 64)));
  }
}

template <bool A_STRIDED, bool B_STRIDED, int TMA>
__device__ __forceinline__ void read_stage_frags(const uint8_t* As, const uint8_t* Bs, const FragAddr& faa,
                                                 const FragAddr& fab, int ks, Frags& f) {
#pragma unroll
  for (int i = 0; i < TMA; ++i) f.a[i] = read_frag<A_STRIDED>(As, faa, ks, i);
#pragma unroll
  for (int j = 0; j < TN; ++j) f.b[j] = read_frag<B_STRIDED>(Bs, fab, ks, j);
}

// Phase fence for the MFMA stream: an empty statement that claims to read and
// rewrite every accumulator.  MFMAs have no side effects, so without it the
// compiler is free to move them across the stage barrier and the fragment
// reads (it did, and then copied fragment registers around the loop).  With
// it, MFMAs issued before the fence stay before it and MFMAs after it stay
// after; it emits no instruction.
__device__ __forceinline__ void mfma_fence(floatx16 (&acc)[TM][TN]) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) asm volatile("" : "+a"(acc[i][j]) :: "memory");
}

// ---- the main loop ---------------------------------------------------------------

// LDS operations of this wave complete, then all waves meet (no wait on
// global memory operations).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt unconstrained
  asm volatile("s_barrier" ::: "memory");
}

// Stores a wave issues for one fp32 output tile of TMA active row blocks
// (store_tile_f32<TMA> issues exactly this many, in or out of range).
template <int TMA>
constexpr int stores_f32() { return TMA * TN * 4; }

// ---- ping-pong main loop -----------------------------------------------------------
//
// The two waves of each SIMD take turns: while one issues a stage's 16
// MFMAs back to back from fragments already in its registers, the other
// reads its fragments of the stage it computes next and issues its share of
// the global->LDS loads.  A load that cannot issue yet, or an LDS read still
// in flight, then holds up only the wave that is not computing, and the
// matrix core sees one uninterrupted MFMA stream after another.  Group g =
// wm (waves 4 g .. 4 g + 3, one per SIMD) owns tile rows 128 g .. (64 g ..
// for a half-height tile).
//
// Steps alternate: in step 2s group 0 computes stage s while group 1 reads
// stage s and loads B of stage s + 3; in step 2s + 1 group 1 computes stage
// s while group 0 reads stage s + 1 and loads A of stage s + 4.  Each step
// ends at a barrier.  Stage s lives in slot s mod 4 (one stage per slot for
// both operands); it is read in steps 2s - 1 and 2s, so its slot is free for
// stage s + 4 from step 2s + 1 on (A) and B of stage s + 3 goes into the
// slot of stage s - 1, free since step 2s - 1.  Group 0 issues every A load
// (4 per wave per odd step), group 1 every B load (4 per wave per even
// step); stage s + 1 must have landed at the barrier that ends step 2s, where
// each wave has at most the 8 loads of the two later stages in flight.
//
// A group's 4 loads per step fill its wave's 4 KB of the operand's 16 KB
// stage tile.

// The load contexts of the group's wave w (0..3) for the stage whose first
// reduction index is q0; load jj (0..3) adds jj * step.
//   Reduction-contiguous (ESZ bytes per element: 2 bf16, 1 e4m3; a chunk is
//   16 bytes either way): load jj covers tile rows 64 w + 16 jj .. + 15;
//   lane i: row 64 w + 16 jj + i / 4, chunk position i mod 4, logical chunk
//   (i mod 4) ^ ((row / 4) mod 4) = (i mod 4) ^ ((i / 16) mod 4).  Chunks
//   past the reduction end read as zero.
//   Reduction-strided: wave w covers tile rows 64 w .. + 63 (128 contiguous
//   bytes of each reduction row; rows 128.. start op.split bytes further,
//   the up half of a gate/up weight), load jj reduction rows 8 jj .. + 7;
//   lane i: reduction row 8 jj + i / 8, chunk position i mod 8, logical
//   chunk (i mod 8) ^ 4 ((i / 16) mod 2).  The range ends at the last
//   reduction row.  WIDE: that row can lie 4 GB or more past this stage (a
//   wgrad expert of 300k rows at k = 7168), which would wrap 32 bits.  A
//   stage reads rows 0..31 of its origin only, so the range then stops at
//   row 63 at most: every valid byte of those rows stays inside it, and it
//   spans at most 2^27 bytes.  Otherwise the host has bounded the whole span
//   below 2^32.
// Lane terms are recomputed per stage (a few VALU ops) rather than hoisted
// and kept live across the unrolled main loop.
template <bool STRIDED, bool WIDE = false, int ESZ = 2>
__device__ __forceinline__ DmaCtx dma_ctx_grp(const Operand& op, int q0, int lane_in, int w) {
  DmaCtx c;
  const int lane = (int)opaque_v((uint32_t)lane_in);
  if constexpr (STRIDED) {
    const int left = op.red - q0;
    int last = left - 1;
    if constexpr (WIDE) last = last < 63 ? last : 63;
    const uint32_t nrec = left > 0 ? (uint32_t)last * op.ld_bytes + op.row_tail : 0u;
    c.rs = make_rsrc(op.origin + (int64_t)q0 * op.ld_bytes, nrec);
    const int chunk = (lane & 7) ^ (4 * ((lane >> 4) & 1));
    c.voff = (uint32_t)(lane >> 3) * op.ld_bytes + (uint32_t)(128 * w + 16 * chunk) + (w >= 2 ? op.split : 0u);
    c.step = 8u * op.ld_bytes;
  } else {
    const uint32_t nrec = q0 < op.red ? (uint32_t)op.rows * op.ld_bytes - (uint32_t)(ESZ * q0) : 0u;
    c.rs = make_rsrc(op.origin + (int64_t)ESZ * q0, nrec);
    const int chunk = (lane & 3) ^ ((lane >> 4) & 3);
    uint32_t v = (uint32_t)(64 * w + (lane >> 2)) * op.ld_bytes + 16u * (uint32_t)chunk;
    if (q0 + (16 / ESZ) * chunk >= op.red) v = kOutOfRange;
    c.voff = v;
    c.step = 16u * op.ld_bytes;
  }
  return c;
}

// (The row step goes through a scalar register: it is uniform, but where the
// two groups' code paths merge the compiler can lose track of that and wrap
// the load in a loop over its distinct values.)
__device__ __forceinline__ void dma_load_grp(const DmaCtx& c, uint8_t* lds_op, int w, int jj) {
  const uint32_t wbase = opaque_s((uint32_t)uniform(w * 4096));
  const uint32_t soff = (uint32_t)uniform((int)(jj * c.step));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rs, LDS_PTR(lds_op + wbase + 1024 * jj), 16, c.voff, soff, 0, 0);
}

// The loads in flight when a tile's ping-pong loop starts: group 0 A of
// stages 0..3, group 1 B of stages 0..2 (16 and 12 per wave).
template <bool A_STRIDED, bool B_STRIDED, bool WIDE = false>
__device__ __attribute__((always_inline)) inline void prologue_loads_pp(
    uint8_t* __restrict__ s0, uint8_t* __restrict__ s1, uint8_t* __restrict__ s2,
    uint8_t* __restrict__ s3, const uint8_t* __restrict__ a_origin,
    const uint8_t* __restrict__ b_origin, Operand A, Operand B, int tid, int wave) {
  A.origin = a_origin;
  B.origin = b_origin;
  const int lane = tid & 63;
  const int w = wave & 3;
  if (wave < 4) {
#define GG_PP_PRO(S, BUF)                                                   \
    {                                                                       \
      const DmaCtx c = dma_ctx_grp<A_STRIDED, WIDE>(A, (S) * BK, lane, w); \
      _Pragma("unroll") for (int jj = 0; jj < 4; ++jj) dma_load_grp(c, (BUF), w, jj); \
    }
    GG_PP_PRO(0, s0) GG_PP_PRO(1, s1) GG_PP_PRO(2, s2) GG_PP_PRO(3, s3)
#undef GG_PP_PRO
  } else {
#define GG_PP_PRO(S, BUF)                                                   \
    {                                                                       \
      const DmaCtx c = dma_ctx_grp<B_STRIDED, WIDE>(B, (S) * BK, lane, w); \
      _Pragma("unroll") for (int jj = 0; jj < 4; ++jj) dma_load_grp(c, (BUF) + OP_BYTES, w, jj); \
    }
    GG_PP_PRO(0, s0) GG_PP_PRO(1, s1) GG_PP_PRO(2, s2)
#undef GG_PP_PRO
  }
}

// Barriers of the ping-pong loops.  The stage buffers are restrict-qualified
// (so that an LDS read need not wait for global->LDS loads into other
// buffers), but here a group reads regions that only the other group's waves
// write.  Seen from one wave, nothing in its own code writes them, and once
// the loop is inlined the compiler takes a barrier (an asm statement) not to
// touch restrict memory whose pointer has not escaped before it, so it would
// be free to reuse a fragment read across iterations.  pp_regions_escape,
// called once at the top of each ping-pong loop, lets every region pointer
// escape into an (empty) asm statement; every later barrier then counts as
// reading and writing them, and no LDS access moves across it.
struct Regions {
  const void* p[8];
};

__device__ __forceinline__ void pp_regions_escape(const Regions& r) {
  asm volatile("" ::"s"((uint32_t)(uintptr_t)r.p[0]), "s"((uint32_t)(uintptr_t)r.p[1]),
               "s"((uint32_t)(uintptr_t)r.p[2]), "s"((uint32_t)(uintptr_t)r.p[3]),
               "s"((uint32_t)(uintptr_t)r.p[4]), "s"((uint32_t)(uintptr_t)r.p[5]),
               "s"((uint32_t)(uintptr_t)r.p[6]), "s"((uint32_t)(uintptr_t)r.p[7])
               : "memory");
}

// s_waitcnt vmcnt(N) expcnt(7) lgkmcnt(0) (N < 64 a count of this wave's
// loads, 64 no wait on loads; vmcnt is 6 bits, the low 4 at [3:0] and the
// high 2 at [15:14]), then barrier.
template <int N>
__device__ __forceinline__ void pp_sync(const Regions&) {
  if constexpr (N < 64) __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  else __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("s_barrier" ::: "memory");
}
constexpr int kNoVm = 64;

// prev_stores: fp32 stores of the previous tile issued after this tile's
// prologue loads (they complete before those loads in the count).
template <bool A_STRIDED, bool B_STRIDED, int TMA, bool WIDE = false>
__device__ __attribute__((always_inline)) inline void mainloop_pp(
    uint8_t* __restrict__ s0, uint8_t* __restrict__ s1, uint8_t* __restrict__ s2,
    uint8_t* __restrict__ s3, const uint8_t* __restrict__ a_origin,
    const uint8_t* __restrict__ b_origin, Operand A, Operand B, int tid, int wave,
    const FragAddr& faa, const FragAddr& fab, floatx16 (&acc)[TM][TN], int prev_stores) {
  A.origin = a_origin;
  B.origin = b_origin;
  const int nk = (A.red + BK - 1) / BK;
  if (nk <= 0) return;
  const int lane = tid & 63;
  const int w = wave & 3;
  const bool g0 = wave < 4;
  const Regions rg = {{s0, s1, s2, s3, s0 + OP_BYTES, s1 + OP_BYTES, s2 + OP_BYTES, s3 + OP_BYTES}};
  pp_regions_escape(rg);
  Frags f0, f1;     // sub-steps 0 and 1 of the stage this wave computes next
  // stage 0 landed: group 0 leaves A of stages 1..3 in flight, group 1 B of
  // stages 1, 2 (plus, after a direct fp32 epilogue, the previous tile's
  // stores, which were issued after these loads)
  if (prev_stores == stores_f32<TM>()) {
    if (g0) pp_sync<12 + stores_f32<TM>()>(rg); else pp_sync<8 + stores_f32<TM>()>(rg);
  } else if (prev_stores == stores_f32<2>()) {
    if (g0) pp_sync<12 + stores_f32<2>()>(rg); else pp_sync<8 + stores_f32<2>()>(rg);
  } else {
    if (g0) pp_sync<12>(rg); else pp_sync<8>(rg);
  }
  if (g0) {
    read_stage_frags<A_STRIDED, B_STRIDED, TMA>(s0, s0 + OP_BYTES, faa, fab, 0, f0);
    read_stage_frags<A_STRIDED, B_STRIDED, TMA>(s0, s0 + OP_BYTES, faa, fab, 1, f1);
  }

#define GG_PP_MFMA()                                                                              \
  {                                                                                               \
    _Pragma("unroll") for (int q = 0; q < TMA * TN; ++q) {                                        \
      const int i = q / TN, j = q % TN;                                                           \
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0.b[j], f0.a[i], acc[i][j], 0, 0, 0); \
    }                                                                                             \
    _Pragma("unroll") for (int q = 0; q < TMA * TN; ++q) {                                        \
      const int i = q / TN, j = q % TN;                                                           \
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1.b[j], f1.a[i], acc[i][j], 0, 0, 0); \
    }                                                                                             \
    mfma_fence(acc);                                                                              \
  }
#define GG_PP_READ(BUF)                                                                           \
  {                                                                                               \
    read_stage_frags<A_STRIDED, B_STRIDED, TMA>(BUF, (BUF) + OP_BYTES, faa, fab, 0, f0);         \
    read_stage_frags<A_STRIDED, B_STRIDED, TMA>(BUF, (BUF) + OP_BYTES, faa, fab, 1, f1);         \
  }
  // Each group runs its own loop (every wave meets the same barriers in the
  // same order: one after each step).  BC: the slot of stage KT; BN: of
  // KT + 1; BP: of KT - 1 (= KT + 3 mod 4).
  if (g0) {
#define GG_PP_STAGE0(BC, BN, BP, KT)                                                              \
  {                                                                                               \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    GG_PP_MFMA()                                     /* step 2 KT: compute stage KT */            \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    pp_sync<8>(rg);                           /* stage KT + 1 landed */                    \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    if ((KT) + 1 < nk) GG_PP_READ(BN)                /* step 2 KT + 1: read stage KT + 1 */       \
    {                                                                                             \
      const DmaCtx ca = dma_ctx_grp<A_STRIDED, WIDE>(A, ((KT) + 4) * BK, lane, w);               \
      _Pragma("unroll") for (int jj = 0; jj < 4; ++jj) dma_load_grp(ca, BC, w, jj);               \
    }                                                                                             \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    pp_sync<kNoVm>(rg);                                   /* fragments in registers */                 \
  }
    for (int kt = 0; kt < nk; kt += 4) {
      GG_PP_STAGE0(s0, s1, s3, kt)
      if (kt + 1 < nk) GG_PP_STAGE0(s1, s2, s0, kt + 1)
      if (kt + 2 < nk) GG_PP_STAGE0(s2, s3, s1, kt + 2)
      if (kt + 3 < nk) GG_PP_STAGE0(s3, s0, s2, kt + 3)
    }
#undef GG_PP_STAGE0
  } else {
#define GG_PP_STAGE1(BC, BN, BP, KT)                                                              \
  {                                                                                               \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    GG_PP_READ(BC)                                   /* step 2 KT: read stage KT */               \
    {                                                                                             \
      const DmaCtx cb = dma_ctx_grp<B_STRIDED, WIDE>(B, ((KT) + 3) * BK, lane, w);               \
      _Pragma("unroll") for (int jj = 0; jj < 4; ++jj) dma_load_grp(cb, (BP) + OP_BYTES, w, jj);  \
    }                                                                                             \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    pp_sync<8>(rg);                           /* stage KT + 1 landed */                    \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    GG_PP_MFMA()                                     /* step 2 KT + 1: compute stage KT */        \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    pp_sync<kNoVm>(rg);                                                                                \
  }
    for (int kt = 0; kt < nk; kt += 4) {
      GG_PP_STAGE1(s0, s1, s3, kt)
      if (kt + 1 < nk) GG_PP_STAGE1(s1, s2, s0, kt + 1)
      if (kt + 2 < nk) GG_PP_STAGE1(s2, s3, s1, kt + 2)
      if (kt + 3 < nk) GG_PP_STAGE1(s3, s0, s2, kt + 3)
    }
#undef GG_PP_STAGE1
  }
#undef GG_PP_READ
#undef GG_PP_MFMA
}

// ---- full-line staging of reduction-contiguous operands (row passes) ---------------
//
// One stage of a reduction-contiguous operand is 64 bytes per tile row: half
// a cache line per row and load.  The row passes (bf16 and fp8) stage their A
// operand two stages at a time instead, so that one load moves 128 contiguous
// bytes (both stages) of 8 tile rows and every line is read whole.
//
// Stage pair j of A holds stages 2j and 2j + 1: tile rows 0..127 in A's
// region of ring slot 2j mod 4, rows 128..255 in that of slot (2j + 1) mod
// 4.  In a region, the 8 rows 8b..8b+7 (of its 128) fill 1 KB block b: the
// first stage's 64 bytes of each row in the block's first 512 bytes, the
// second stage's in the other 512, each row at 64 (r mod 8) with its 16-byte
// chunks swizzled c ^ ((r / 4) mod 4) as in the single-stage layout
// (fragment reads stay bank-conflict-free).  B keeps one stage per slot,
// whether reduction-strided (forward) or -contiguous (dgrad, whose B is the
// weight stream: pairing it too measured slower, as it then has less time to
// arrive).

struct DmaPair {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t voff0;     // lane offset of loads 0 and 2
  uint32_t voff1;     // of loads 1 and 3 (their rows' swizzle differs by 2)
  uint32_t step;      // 8 rows (scalar offset per load)
};

// The 4 loads a wave issues for the stage pair of A whose first reduction
// element is q0 (ESZ bytes per element: a stage is 64 bytes of a row, 32 bf16
// or 64 e4m3 values).  Load jj of
// wave w covers tile rows 32 w + 8 jj .. + 7 (block 4 (w mod 4) + jj of
// region w / 4); lane i: stage i / 32 of the pair, row 32 w + 8 jj + (i mod
// 32) / 4, chunk position i mod 4, logical chunk (i mod 4) ^ ((row / 4) mod
// 4).  Values outside [0, red) and rows past the tile read as zero.
template <int ESZ = 2>
__device__ __forceinline__ DmaPair dma_pair(const Operand& op, int q0, int tid) {
  const int lane = (int)opaque_v((uint32_t)(tid & 63));
  const int w = tid >> 6;
  DmaPair c;
  const uint32_t nrec = q0 < op.red ? (uint32_t)op.rows * op.ld_bytes - (uint32_t)(ESZ * q0) : 0u;
  c.rs = make_rsrc(op.origin + (int64_t)ESZ * q0, nrec);
  const int rin = (lane & 31) >> 2;
  const int sw = rin >> 2;                           // ((32 w + rin) / 4) mod 4 for loads 0 and 2
  const int kl = q0 + (64 / ESZ) * (lane >> 5);
  const int k0 = kl + (16 / ESZ) * ((lane & 3) ^ sw);
  const int k1 = kl + (16 / ESZ) * ((lane & 3) ^ sw ^ 2);
  const uint32_t rowoff = (uint32_t)(32 * w + rin) * op.ld_bytes;
  c.voff0 = k0 < op.red ? rowoff + (uint32_t)(ESZ * (k0 - q0)) : kOutOfRange;
  c.voff1 = k1 < op.red ? rowoff + (uint32_t)(ESZ * (k1 - q0)) : kOutOfRange;
  c.step = 8u * op.ld_bytes;
  return c;
}

__device__ __forceinline__ void dma_load_pair(const DmaPair& c, uint8_t* region, int wave, int jj) {
  const uint32_t wbase = opaque_s((uint32_t)uniform((wave & 3) * 4096));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rs, LDS_PTR(region + wbase + 1024 * jj), 16,
                                           (jj & 1) ? c.voff1 : c.voff0, jj * c.step, 0, 0);
}

// dma_load_pair with its row step moved to a scalar register: the value is
// uniform, but where the two groups' code paths merge the compiler can lose
// track of that and wrap the load in a loop over its distinct values.
__device__ __forceinline__ void dma_load_pair_s(const DmaPair& c, uint8_t* region, int wave, int jj) {
  const uint32_t wbase = opaque_s((uint32_t)uniform((wave & 3) * 4096));
  const uint32_t soff = (uint32_t)uniform((int)(jj * c.step));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rs, LDS_PTR(region + wbase + 1024 * jj), 16,
                                           (jj & 1) ? c.voff1 : c.voff0, soff, 0, 0);
}

// Fragment addresses in the pair layout for a wave slice starting at tile
// row r0 (a multiple of 64; the slice lies in one region): chunk 2 ks + l /
// 32 of row r0 + l % 32.  Fragment i adds 4096, the second stage 512.
__device__ __forceinline__ FragAddr frag_addr_pair(int r0, int lane) {
  FragAddr f;
  const int rr = (r0 & 127) + (lane & 31);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int chunk = (2 * ks + (lane >> 5)) ^ ((rr >> 2) & 3);
    f.o[ks] = (uint32_t)((rr >> 3) * 1024 + (rr & 7) * 64 + 16 * chunk);
  }
  return f;
}

__device__ __forceinline__ bf16x8 read_frag_pair(const uint8_t* region, const FragAddr& fa, int ks, int i,
                                                 int par) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(region + fa.o[ks] +
                                                                     (uint32_t)(i * 4096 + par * 512)));
}

// ---- ping-pong main loop with A in the pair layout (bf16 row passes) ----------------
//
// The ping-pong schedule above, with the reduction-contiguous A operand
// staged two stages at a time in the pair layout (whole cache lines), B one
// stage per slot.  Group g's rows of A pair p (stages 2p, 2p + 1) sit in the
// A region of slot (2p + g) mod 4, and group g loads them itself (the pair
// loads of its waves); B of a stage is loaded by one group's 4 waves.  Over
// each pair of stages s = 2j, 2j + 1 (steps 4j .. 4j + 3):
//   step 4j     group 0 computes stage 2j;     group 1 reads stage 2j and
//               loads its half of A pair j + 1
//   step 4j + 1 group 1 computes stage 2j;     group 0 reads stage 2j + 1 and
//               loads B of stage 2j + 4
//   step 4j + 2 group 0 computes stage 2j + 1; group 1 reads stage 2j + 1
//               and loads B of stage 2j + 3
//   step 4j + 3 group 1 computes stage 2j + 1; group 0 reads stage 2j + 2
//               and loads its half of A pair j + 2
// Every load goes into a region whose earlier contents were last read at
// least one barrier before, and lands 3 to 6 steps later; the barrier that
// precedes its first reader waits for it (vmcnt(4): the group's one later
// batch of 4 may still be in flight).  For a half-height tile every wave's
// rows lie in group 0's region (ha = 0); group 1's pair loads then read only
// rows past the tile, which land as zeros and are never read.

// Loads in flight when the loop starts, in this order: group 0 B of stage 0,
// its half of A pair 0, B of stage 2, its half of A pair 1; group 1 its half
// of A pair 0, B of stage 1.
template <bool B_STRIDED>
__device__ __attribute__((always_inline)) inline void prologue_loads_pp_pair(
    uint8_t* __restrict__ a0, uint8_t* __restrict__ a1, uint8_t* __restrict__ a2, uint8_t* __restrict__ a3,
    uint8_t* __restrict__ b0, uint8_t* __restrict__ b1, uint8_t* __restrict__ b2,
    const uint8_t* __restrict__ a_origin, const uint8_t* __restrict__ b_origin, Operand A, Operand B, int tid,
    int wave) {
  A.origin = a_origin;
  B.origin = b_origin;
  const int lane = tid & 63;
  const int w = wave & 3;
  if (wave < 4) {
    {
      const DmaCtx c = dma_ctx_grp<B_STRIDED>(B, 0, lane, w);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) dma_load_grp(c, b0, w, jj);
    }
    {
      const DmaPair c = dma_pair(A, 0, tid);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) dma_load_pair_s(c, a0, wave, jj);
    }
    {
      const DmaCtx c = dma_ctx_grp<B_STRIDED>(B, 2 * BK, lane, w);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) dma_load_grp(c, b2, w, jj);
    }
    {
      const DmaPair c = dma_pair(A, 2 * BK, tid);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) dma_load_pair_s(c, a2, wave, jj);
    }
  } else {
    {
      const DmaPair c = dma_pair(A, 0, tid);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) dma_load_pair_s(c, a1, wave, jj);
    }
    {
      const DmaCtx c = dma_ctx_grp<B_STRIDED>(B, BK, lane, w);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) dma_load_grp(c, b1, w, jj);
    }
  }
}

template <bool B_STRIDED, int TMA>
__device__ __attribute__((always_inline)) inline void mainloop_pp_pair(
    uint8_t* __restrict__ a0, uint8_t* __restrict__ a1, uint8_t* __restrict__ a2, uint8_t* __restrict__ a3,
    uint8_t* __restrict__ b0, uint8_t* __restrict__ b1, uint8_t* __restrict__ b2, uint8_t* __restrict__ b3,
    const uint8_t* __restrict__ a_origin, const uint8_t* __restrict__ b_origin, Operand A, Operand B, int tid,
    int wave, int ha, const FragAddr& faa, const FragAddr& fab, floatx16 (&acc)[TM][TN],
    int prev_stores) {
  A.origin = a_origin;
  B.origin = b_origin;
  const int nk = (A.red + BK - 1) / BK;
  if (nk <= 0) return;
  const int lane = tid & 63;
  const int w = wave & 3;
  const bool g0 = wave < 4;
  const Regions rg = {{a0, a1, a2, a3, b0, b1, b2, b3}};
  pp_regions_escape(rg);
  Frags f0, f1;
  // group 0: B of stage 0 and its half of A pair 0 landed (its other 8 loads
  // and the previous tile's direct stores, issued after them, may be in
  // flight); group 1 waits at the next barrier
  if (prev_stores == stores_f32<TM>()) {
    if (g0) pp_sync<8 + stores_f32<TM>()>(rg); else pp_sync<kNoVm>(rg);
  } else if (prev_stores == stores_f32<2>()) {
    if (g0) pp_sync<8 + stores_f32<2>()>(rg); else pp_sync<kNoVm>(rg);
  } else {
    if (g0) pp_sync<8>(rg); else pp_sync<kNoVm>(rg);
  }

#define GG_RA(U) ((U) < 2 ? (ha ? a1 : a0) : (ha ? a3 : a2))
#define GG_RB(U) ((U) == 0 ? b0 : (U) == 1 ? b1 : (U) == 2 ? b2 : b3)
#define GG_PP_READ(U)                                                                             \
  {                                                                                               \
    _Pragma("unroll") for (int i = 0; i < TMA; ++i) f0.a[i] = read_frag_pair(GG_RA(U), faa, 0, i, (U) & 1); \
    _Pragma("unroll") for (int j = 0; j < TN; ++j) f0.b[j] = read_frag<B_STRIDED>(GG_RB(U), fab, 0, j);    \
    _Pragma("unroll") for (int i = 0; i < TMA; ++i) f1.a[i] = read_frag_pair(GG_RA(U), faa, 1, i, (U) & 1); \
    _Pragma("unroll") for (int j = 0; j < TN; ++j) f1.b[j] = read_frag<B_STRIDED>(GG_RB(U), fab, 1, j);    \
  }
#define GG_PP_MFMA()                                                                              \
  {                                                                                               \
    _Pragma("unroll") for (int q = 0; q < TMA * TN; ++q) {                                        \
      const int i = q / TN, j = q % TN;                                                           \
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0.b[j], f0.a[i], acc[i][j], 0, 0, 0); \
    }                                                                                             \
    _Pragma("unroll") for (int q = 0; q < TMA * TN; ++q) {                                        \
      const int i = q / TN, j = q % TN;                                                           \
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1.b[j], f1.a[i], acc[i][j], 0, 0, 0); \
    }                                                                                             \
    mfma_fence(acc);                                                                              \
  }
// B of stage Q into slot U (one group's 4 waves)
#define GG_PP_LOAD_B(U, Q)                                                                        \
  {                                                                                               \
    const DmaCtx cb = dma_ctx_grp<B_STRIDED>(B, (Q) * BK, lane, w);                               \
    _Pragma("unroll") for (int jj = 0; jj < 4; ++jj) dma_load_grp(cb, GG_RB(U), w, jj);            \
  }
// this wave's rows of the A pair whose first stage is Q, into region R
#define GG_PP_LOAD_A(R, Q)                                                                        \
  {                                                                                               \
    const DmaPair cp = dma_pair(A, (Q) * BK, tid);                                                \
    _Pragma("unroll") for (int jj = 0; jj < 4; ++jj) dma_load_pair_s(cp, (R), wave, jj);          \
  }

  if (g0) {
    // step -1: read stage 0
    GG_PP_READ(0)
    __builtin_amdgcn_sched_barrier(0);
    pp_sync<kNoVm>(rg);
    // stage KT = kt + U: compute it, then read stage KT + 1 and load (U even)
    // B of stage KT + 4 into slot U or (U odd) this group's half of the A
    // pair of stages KT + 3, KT + 4 into slot (U + 3) mod 4
#define GG_PP_STAGE0(U, KT)                                                                       \
  {                                                                                               \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    GG_PP_MFMA()                                                                                  \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    if ((U) & 1) pp_sync<4>(rg); else pp_sync<kNoVm>(rg);                                      \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    if ((KT) + 1 < nk) GG_PP_READ(((U) + 1) & 3)                                                  \
    if (((U) & 1) == 0) GG_PP_LOAD_B(U, (KT) + 4)                                                 \
    else GG_PP_LOAD_A((U) == 1 ? a0 : a2, (KT) + 3)                                               \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    pp_sync<kNoVm>(rg);                                                                                \
  }
    for (int kt = 0; kt < nk; kt += 4) {
      GG_PP_STAGE0(0, kt)
      if (kt + 1 < nk) GG_PP_STAGE0(1, kt + 1)
      if (kt + 2 < nk) GG_PP_STAGE0(2, kt + 2)
      if (kt + 3 < nk) GG_PP_STAGE0(3, kt + 3)
    }
#undef GG_PP_STAGE0
  } else {
    // step -1: this group's half of A pair 0 landed (B of stage 1 may be in
    // flight, and the previous tile's direct stores after it)
    __builtin_amdgcn_sched_barrier(0);
    if (prev_stores == stores_f32<TM>()) pp_sync<4 + stores_f32<TM>()>(rg);
    else if (prev_stores == stores_f32<2>()) pp_sync<4 + stores_f32<2>()>(rg);
    else pp_sync<4>(rg);
    // stage KT = kt + U: read it and load (U even) this group's half of the A
    // pair of stages KT + 2, KT + 3 into slot (U + 3) mod 4 or (U odd) B of
    // stage KT + 2 into slot (U + 2) mod 4; then compute it
#define GG_PP_STAGE1(U, KT)                                                                       \
  {                                                                                               \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    GG_PP_READ(U)                                                                                 \
    if (((U) & 1) == 0) GG_PP_LOAD_A((U) == 0 ? a3 : a1, (KT) + 2)                                \
    else GG_PP_LOAD_B(((U) + 2) & 3, (KT) + 2)                                                    \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    if (((U) & 1) == 0) pp_sync<4>(rg); else pp_sync<kNoVm>(rg);                               \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    GG_PP_MFMA()                                                                                  \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    if ((U) & 1) pp_sync<4>(rg); else pp_sync<kNoVm>(rg);                                      \
  }
    for (int kt = 0; kt < nk; kt += 4) {
      GG_PP_STAGE1(0, kt)
      if (kt + 1 < nk) GG_PP_STAGE1(1, kt + 1)
      if (kt + 2 < nk) GG_PP_STAGE1(2, kt + 2)
      if (kt + 3 < nk) GG_PP_STAGE1(3, kt + 3)
    }
#undef GG_PP_STAGE1
  }
#undef GG_PP_LOAD_A
#undef GG_PP_LOAD_B
#undef GG_PP_MFMA
#undef GG_PP_READ
#undef GG_RB
#undef GG_RA
}

// ---- fp8 (e4m3) block-scaled main loop ----------------------------------------------
//
// The same tile engine on bytes: a stage is 64 e4m3 values (64 bytes) of
// each of the 256 tile rows of X and W, i.e. exactly the bytes of a bf16
// stage, in the same reduction-contiguous LDS layout; one
// v_mfma_scale_f32_32x32x64_f8f6f4 per 32 x 32 block consumes a stage in
// the time two bf16 MFMAs take, so a stage does twice the FLOPs in the same
// cycles and bytes.  The MFMA applies the block scales itself: each lane
// hands it one E8M0 byte (2^(e - 127)) for its row of either operand, and a
// 64-deep MFMA lies inside one 128-value scale block, so the byte is the
// row's scale for that block.
//
// Packed scales.  For every 256-row tile of X (an expert's row tile rt, in
// the order of the experts; masked: expert e's tiles at e * ceil(max_m /
// 256)) and every 256-column tile of W (expert e, column tile ct at e *
// ceil(N / 256) + ct), the scales of k-block kb are 256 bytes at
// ((tile * kblocks) + kb) * 256, tile row r at byte 128 (r / 128) + 4 (r mod
// 32) + (r / 32) mod 4.  So the 4 scales a lane needs (its row in each of
// the wave's four 32-row blocks) are one dword.  Per k-block, wave 0 copies
// the tile's 256 X-scale bytes and wave 1 its 256 W-scale bytes into a
// 2-slot LDS ring with one direct-to-LDS dword load each, issued two k-blocks
// ahead with the stage loads; every lane reads its two dwords once per
// k-block.
typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int BK8 = 64;             // e4m3 values per stage
constexpr int kScaleSlot = 512;     // LDS bytes of one k-block's scales (X, then W)

// Fragment i of a stage: 32 bytes of row 32 i + l % 32 -- the two 16-byte
// chunks the bf16 sub-steps read (chunks l / 32 and 2 + l / 32).  Which
// reduction values a lane holds does not matter as long as both operands
// agree, and they share the layout.
__device__ __forceinline__ i32x8 read_frag8(const uint8_t* lds, const FragAddr& fa, int i) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(lds + fa.o[0] + (uint32_t)(i * 32 * 64));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(lds + fa.o[1] + (uint32_t)(i * 32 * 64));
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One scaled MFMA of block (i, j): source A is the W fragment wf (output
// columns) with scale byte j of sb, source B the X fragment xf (rows) with
// byte i of sa, so the block holds C^T as in the bf16 loop.  The byte
// selects are immediates, hence the switch (folded once the callers' loops
// are unrolled).
__device__ __forceinline__ floatx16 mfma8(int i, int j, const i32x8& wf, const i32x8& xf, floatx16 c,
                                          uint32_t sa, uint32_t sb) {
#define GG_MF8(I, J) \
  case (I) * 2 + (J): return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf, xf, c, 0, 0, J, (int)sb, I, (int)sa);
  switch (i * 2 + j) {
    GG_MF8(0, 0) GG_MF8(0, 1) GG_MF8(1, 0) GG_MF8(1, 1)
    GG_MF8(2, 0) GG_MF8(2, 1) GG_MF8(3, 0) GG_MF8(3, 1)
  }
#undef GG_MF8
  return c;
}

// Wave 0 copies the X scales, wave 1 the W scales of k-block kb into an LDS
// slot (out-of-range blocks land as zeros and are never read).
__device__ __forceinline__ void scale_load(const uint8_t* __restrict__ sa_tile,
                                           const uint8_t* __restrict__ sb_tile, uint32_t nbytes, int kb,
                                           uint8_t* slot, int wave, int lane) {
  if (wave < 2) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(wave == 0 ? sa_tile : sb_tile, nbytes);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_PTR(slot + (wave == 0 ? 0 : 256)), 4,
                                             opaque_v((uint32_t)lane * 4u), (uint32_t)kb * 256u, 0, 0);
  }
}

// This lane's scale dwords for one k-block from its LDS slot, shifted so
// that byte i (X) / byte j (W) is the scale of the wave's block i / j.
template <int TMA>
__device__ __forceinline__ void scale_read(const uint8_t* slot, int wm, int wn, int lane, uint32_t& sa,
                                           uint32_t& sb) {
  const int wa = TMA == 2 ? 0 : wm;
  sa = *reinterpret_cast<const uint32_t*>(slot + 4 * (32 * wa + (lane & 31)));
  sb = *reinterpret_cast<const uint32_t*>(slot + 256 + 4 * (32 * (wn >> 1) + (lane & 31)));
  if (TMA == 2) sa >>= 16 * wm;
  sb >>= 16 * (wn & 1);
}

// Fragment i of a stage of X in the pair layout (the two chunks read_frag8
// reads, at the pair layout's offsets).
__device__ __forceinline__ i32x8 read_frag8_pair(const uint8_t* region, const FragAddr& fa, int i, int par) {
  const uint32_t d = (uint32_t)(i * 4096 + par * 512);
  const u32x4 lo = *reinterpret_cast<const u32x4*>(region + fa.o[0] + d);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(region + fa.o[1] + d);
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---- fp8 ping-pong main loop ---------------------------------------------------------
//
// The bf16 row passes' paired ping-pong schedule on e4m3 operands: X (A) in
// the pair layout, W (B) one stage per slot, each group's waves taking turns
// with a stage's 8 scaled MFMAs.  K is a multiple of 128, so A pair p (stages
// 2p, 2p + 1) is exactly scale k-block p.  Waves 0 and 1 load the k-block's
// X and W scale bytes into slot p mod 2 of the LDS scale ring as the first
// load of the batch that brings group 0's half of the A pair, so the waits of
// the bf16 schedule (vmcnt(4) where a group's next batch may still be in
// flight) cover them unchanged; every wave reads its two scale dwords when it
// reads the first stage of a k-block and keeps them for both stages.  The
// prologue issues the first two k-blocks' scales ahead of everything else.

// Loads in flight when the loop starts, in this order: group 0 (waves 0, 1
// only) the scales of k-blocks 0 and 1, B of stage 0, its half of A pair 0,
// B of stage 2, its half of A pair 1; group 1 its half of A pair 0, B of
// stage 1.
__device__ __attribute__((always_inline)) inline void prologue_loads8_pp(
    uint8_t* __restrict__ a0, uint8_t* __restrict__ a1, uint8_t* __restrict__ a2,
    uint8_t* __restrict__ b0, uint8_t* __restrict__ b1, uint8_t* __restrict__ b2, uint8_t* __restrict__ sc,
    const uint8_t* __restrict__ a_origin, const uint8_t* __restrict__ b_origin,
    const uint8_t* __restrict__ sa_tile, const uint8_t* __restrict__ sb_tile, uint32_t sc_bytes, Operand A,
    Operand B, int tid, int wave) {
  A.origin = a_origin;
  B.origin = b_origin;
  const int lane = tid & 63;
  const int w = wave & 3;
  if (wave < 4) {
    scale_load(sa_tile, sb_tile, sc_bytes, 0, sc, wave, lane);
    scale_load(sa_tile, sb_tile, sc_bytes, 1, sc + kScaleSlot, wave, lane);
    {
      const DmaCtx c = dma_ctx_grp<false, false, 1>(B, 0, lane, w);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) dma_load_grp(c, b0, w, jj);
    }
    {
      const DmaPair c = dma_pair<1>(A, 0, tid);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) dma_load_pair_s(c, a0, wave, jj);
    }
    {
      const DmaCtx c = dma_ctx_grp<false, false, 1>(B, 2 * BK8, lane, w);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) dma_load_grp(c, b2, w, jj);
    }
    {
      const DmaPair c = dma_pair<1>(A, 2 * BK8, tid);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) dma_load_pair_s(c, a2, wave, jj);
    }
  } else {
    {
      const DmaPair c = dma_pair<1>(A, 0, tid);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) dma_load_pair_s(c, a1, wave, jj);
    }
    {
      const DmaCtx c = dma_ctx_grp<false, false, 1>(B, BK8, lane, w);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) dma_load_grp(c, b1, w, jj);
    }
  }
}

template <int TMA>
__device__ __attribute__((always_inline)) inline void mainloop8_pp(
    uint8_t* __restrict__ a0, uint8_t* __restrict__ a1, uint8_t* __restrict__ a2, uint8_t* __restrict__ a3,
    uint8_t* __restrict__ b0, uint8_t* __restrict__ b1, uint8_t* __restrict__ b2, uint8_t* __restrict__ b3,
    uint8_t* __restrict__ sc, const uint8_t* __restrict__ a_origin, const uint8_t* __restrict__ b_origin,
    const uint8_t* __restrict__ sa_tile, const uint8_t* __restrict__ sb_tile, uint32_t sc_bytes, Operand A,
    Operand B, int tid, int wave, int wm, int wn, int ha, const FragAddr& faa, const FragAddr& fab,
    floatx16 (&acc)[TM][TN]) {
  A.origin = a_origin;
  B.origin = b_origin;
  const int nk = (A.red + BK8 - 1) / BK8;           // even: K is a multiple of 128
  if (nk <= 0) return;
  const int lane = tid & 63;
  const int w = wave & 3;
  const bool g0 = wave < 4;
  const Regions rg = {{a0, a1, a2, a3, b0, b1, b2, b3}};
  pp_regions_escape(rg);
  const Regions rs = {{sc, sc, sc, sc, sc, sc, sc, sc}};
  pp_regions_escape(rs);
  i32x8 fa[TMA], fb[TN];
  uint32_t sa = 0, sb = 0;
  // group 0: the scales, B of stage 0 and its half of A pair 0 landed (the
  // last 8 loads may be in flight); group 1 waits at the next barrier
  if (g0) pp_sync<8>(rg); else pp_sync<kNoVm>(rg);

#define GG8_RA(U) ((U) < 2 ? (ha ? a1 : a0) : (ha ? a3 : a2))
#define GG8_RB(U) ((U) == 0 ? b0 : (U) == 1 ? b1 : (U) == 2 ? b2 : b3)
// read stage U's fragments (and, for the first stage of a k-block, its
// scales from slot (U / 2) mod 2 of the ring)
#define GG8_PP_READ(U)                                                                            \
  {                                                                                               \
    if (((U) & 1) == 0) scale_read<TMA>(sc + (((U) >> 1) & 1) * kScaleSlot, wm, wn, lane, sa, sb); \
    _Pragma("unroll") for (int i = 0; i < TMA; ++i) fa[i] = read_frag8_pair(GG8_RA(U), faa, i, (U) & 1); \
    _Pragma("unroll") for (int j = 0; j < TN; ++j) fb[j] = read_frag8(GG8_RB(U), fab, j);        \
  }
#define GG8_PP_MFMA()                                                                             \
  {                                                                                               \
    _Pragma("unroll") for (int q = 0; q < TMA * TN; ++q) {                                        \
      const int i = q / TN, j = q % TN;                                                           \
      acc[i][j] = mfma8(i, j, fb[j], fa[i], acc[i][j], sa, sb);                                   \
    }                                                                                             \
    mfma_fence(acc);                                                                              \
  }
#define GG8_PP_LOAD_B(U, Q)                                                                       \
  {                                                                                               \
    const DmaCtx cb = dma_ctx_grp<false, false, 1>(B, (Q) * BK8, lane, w);                        \
    _Pragma("unroll") for (int jj = 0; jj < 4; ++jj) dma_load_grp(cb, GG8_RB(U), w, jj);           \
  }
#define GG8_PP_LOAD_A(R, Q)                                                                       \
  {                                                                                               \
    const DmaPair cp = dma_pair<1>(A, (Q) * BK8, tid);                                            \
    _Pragma("unroll") for (int jj = 0; jj < 4; ++jj) dma_load_pair_s(cp, (R), wave, jj);          \
  }

  if (g0) {
    GG8_PP_READ(0)
    __builtin_amdgcn_sched_barrier(0);
    pp_sync<kNoVm>(rg);
    // stage KT = kt + U: compute it, then read stage KT + 1 and load (U even)
    // B of stage KT + 4 into slot U or (U odd) the scales of k-block
    // (KT + 3) / 2 and this group's half of its A pair into slot (U + 3) mod 4.
    // The read is unconditional: after the last stage it reads LDS that
    // nothing uses (under a condition the compiler kept the old and the new
    // fragments live across it, copying them and spilling).
#define GG8_PP_STAGE0(U, KT)                                                                      \
  {                                                                                               \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    GG8_PP_MFMA()                                                                                 \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    if ((U) & 1) pp_sync<4>(rg); else pp_sync<kNoVm>(rg);                                          \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    GG8_PP_READ(((U) + 1) & 3)                                                                    \
    if (((U) & 1) == 0) GG8_PP_LOAD_B(U, (KT) + 4)                                                \
    else {                                                                                        \
      scale_load(sa_tile, sb_tile, sc_bytes, ((KT) + 3) / 2, sc + ((((KT) + 3) / 2) & 1) * kScaleSlot, \
                 wave, lane);                                                                     \
      GG8_PP_LOAD_A((U) == 1 ? a0 : a2, (KT) + 3)                                                 \
    }                                                                                             \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    pp_sync<kNoVm>(rg);                                                                           \
  }
    for (int kt = 0; kt < nk; kt += 4) {
      GG8_PP_STAGE0(0, kt)
      GG8_PP_STAGE0(1, kt + 1)
      if (kt + 2 < nk) {
        GG8_PP_STAGE0(2, kt + 2)
        GG8_PP_STAGE0(3, kt + 3)
      }
    }
#undef GG8_PP_STAGE0
  } else {
    // this group's half of A pair 0 landed (B of stage 1 may be in flight)
    __builtin_amdgcn_sched_barrier(0);
    pp_sync<4>(rg);
    // stage KT = kt + U: read it and load (U even) this group's half of the A
    // pair of stages KT + 2, KT + 3 into slot (U + 3) mod 4 or (U odd) B of
    // stage KT + 2 into slot (U + 2) mod 4; then compute it
#define GG8_PP_STAGE1(U, KT)                                                                      \
  {                                                                                               \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    GG8_PP_READ(U)                                                                                \
    if (((U) & 1) == 0) GG8_PP_LOAD_A((U) == 0 ? a3 : a1, (KT) + 2)                               \
    else GG8_PP_LOAD_B(((U) + 2) & 3, (KT) + 2)                                                   \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    if (((U) & 1) == 0) pp_sync<4>(rg); else pp_sync<kNoVm>(rg);                                   \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    GG8_PP_MFMA()                                                                                 \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    if ((U) & 1) pp_sync<4>(rg); else pp_sync<kNoVm>(rg);                                          \
  }
    for (int kt = 0; kt < nk; kt += 4) {
      GG8_PP_STAGE1(0, kt)
      GG8_PP_STAGE1(1, kt + 1)
      if (kt + 2 < nk) {
        GG8_PP_STAGE1(2, kt + 2)
        GG8_PP_STAGE1(3, kt + 3)
      }
    }
#undef GG8_PP_STAGE1
  }
#undef GG8_PP_LOAD_A
#undef GG8_PP_LOAD_B
#undef GG8_PP_MFMA
#undef GG8_PP_READ
#undef GG8_RB
#undef GG8_RA
}

// ---- epilogue --------------------------------------------------------------------

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (round to nearest even) packed in one dword, low
// half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  floatx2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// fp32 output straight from the accumulators.  Accumulator block (i, j)
// holds C^T: element v of lane l is output row 32 TMA wm + 32 i + l % 32 and
// output column 64 wn + 32 j + 8 (v / 4) + 4 (l / 32) + v % 4, so each lane
// stores 4 consecutive columns (16 bytes) at a time.  Stores go through a
// buffer resource ending at the tile's last valid element: rows past the
// valid ones are dropped by the range check, and a group of 8 columns past
// the valid ones (cols is a multiple of 8) is sent out of range.
template <int TMA>
__device__ __forceinline__ void store_tile_f32(uint8_t* cbase, uint32_t ldc_bytes, int rows, int cols,
                                               int wm, int wn, int lane, const floatx16 (&acc)[TM][TN]) {
  constexpr uint32_t esz = 4;
  const uint32_t nrec = (uint32_t)(rows - 1) * ldc_bytes + (uint32_t)cols * esz;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(cbase, nrec);
  const uint32_t lane_off = opaque_v((uint32_t)(32 * TMA * wm + (lane & 31)) * ldc_bytes +
                                     (uint32_t)(64 * wn + 4 * (lane >> 5)) * esz);
#pragma unroll
  for (int i = 0; i < TMA; ++i) {
    const uint32_t voff = lane_off + (uint32_t)(32 * i) * ldc_bytes;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const floatx16& a = acc[i][j];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int col8 = 64 * wn + 32 * j + 8 * rr;       // first of 8 columns, wave-uniform
        const uint32_t imm = (uint32_t)(32 * j + 8 * rr) * esz;
        // Column groups past the last valid column are stored out of range
        // (dropped) rather than skipped, so every tile of a shape issues the
        // same number of stores (the next tile's first wait counts them).
        // Built as a float vector and bit-cast whole: a u32x4 built from
        // per-element bit casts of accumulator values was miscompiled by
        // this hipcc (every lane of the vector got element 0).
        floatx4 v = {a[4 * rr + 0], a[4 * rr + 1], a[4 * rr + 2], a[4 * rr + 3]};
        const uint32_t off = col8 < cols ? voff + imm : kOutOfRange;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off, 0, 0);
      }
    }
  }
}

// Output through LDS: the bf16 epilogue, and the scaled form (alpha, beta)
// of either output type.  Packing or combining needs the values in ordinary
// registers; moving all 128 accumulators there at once overflows them, so
// each wave instead writes one 32 x 64 fp32 slab (block row i) from its
// accumulator registers into its own LDS region (rows padded by 16 bytes so
// the 16 rows a write touches fall on distinct banks) and reads back 8
// consecutive values per lane.  Those become alpha * v + beta * c, with c the
// 8 prior output values of the same elements (read only when beta != 0,
// through the same range-checked resource: out of range reads as zero),
// then one rounding to the output type; 8 lanes cover a slab row's 64
// contiguous output columns.  Row and column predication as in
// store_tile_f32.  `slab` is this wave's LDS region (>= 32 * 272 bytes),
// free for the epilogue.
constexpr int kSlabPitch = 64 * 4 + 16;

template <int TMA, bool OUT_F32, bool SCALED>
__device__ __forceinline__ void store_tile_lds(uint8_t* cbase, uint32_t ldc_bytes, int rows, int cols,
                                               int wm, int wn, int lane, const floatx16 (&acc)[TM][TN],
                                               uint8_t* slab, float alpha, float beta,
                                               const uint16_t* bias = nullptr,
                                               const float* bscale = nullptr) {
  constexpr uint32_t esz = OUT_F32 ? 4 : 2;
  const uint32_t nrec = (uint32_t)(rows - 1) * ldc_bytes + (uint32_t)cols * esz;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(cbase, nrec);
  // Lane-dependent offsets, recomputed per call rather than hoisted out of
  // the tile loop (where they would stay live across the main loop):
  // write: slab row l % 32, its 4 columns 4 (l / 32) of each 8-column group;
  // read: 8 consecutive columns 8 (l % 8) of slab rows l / 8 + 8 q.
  const uint32_t wslab = opaque_v((uint32_t)((lane & 31) * kSlabPitch + 16 * (lane >> 5)));
  const uint32_t rslab = opaque_v((uint32_t)((lane >> 3) * kSlabPitch + 32 * (lane & 7)));
  const int gcol = 64 * wn + 8 * (lane & 7);
  const bool col_ok = gcol < cols;
  const uint32_t gbase = col_ok ? opaque_v((uint32_t)(32 * TMA * wm + (lane >> 3)) * ldc_bytes +
                                           (uint32_t)gcol * esz)
                                : kOutOfRange;
#pragma unroll
  for (int i = 0; i < TMA; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        floatx4 v = {acc[i][j][4 * rr + 0], acc[i][j][4 * rr + 1], acc[i][j][4 * rr + 2], acc[i][j][4 * rr + 3]};
        *reinterpret_cast<floatx4*>(slab + wslab + 4 * (32 * j + 8 * rr)) = v;
      }
    // LDS operations of one wave complete in order: the reads see the writes.
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      floatx4 lo = *reinterpret_cast<const floatx4*>(slab + rslab + 8 * q * kSlabPitch);
      floatx4 hi = *reinterpret_cast<const floatx4*>(slab + rslab + 8 * q * kSlabPitch + 16);
      // rows 32 TMA wm + 32 i + l / 8 + 8 q (out of range stays out of range)
      const uint32_t voff = gbase + (uint32_t)(32 * i + 8 * q) * ldc_bytes;
      if constexpr (SCALED) {
        lo = lo * alpha;
        hi = hi * alpha;
        if (beta != 0.0f) {
          floatx4 clo, chi;
          if constexpr (OUT_F32) {
            clo = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0));
            chi = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16, 0, 0));
          } else {
            // 8 bf16 values: each is the high half of its fp32 pattern
            const u32x4 c = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0));
            clo = floatx4{__builtin_bit_cast(float, c[0] << 16), __builtin_bit_cast(float, c[0] & 0xFFFF0000u),
                          __builtin_bit_cast(float, c[1] << 16), __builtin_bit_cast(float, c[1] & 0xFFFF0000u)};
            chi = floatx4{__builtin_bit_cast(float, c[2] << 16), __builtin_bit_cast(float, c[2] & 0xFFFF0000u),
                          __builtin_bit_cast(float, c[3] << 16), __builtin_bit_cast(float, c[3] & 0xFFFF0000u)};
          }
          lo = lo + clo * beta;
          hi = hi + chi * beta;
        }
        if (bias) {
          // + s[row] * bias[col]: the tile's bias row (its 8 columns of this
          // lane) and the row's factor, both through range-checked
          // resources (columns past cols and rows past rows read as zero)
          const uint32_t boff = col_ok ? opaque_v((uint32_t)gcol * 2u) : kOutOfRange;
          const u32x4 b = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(bias, (uint32_t)cols * 2u), boff, 0, 0));
          const floatx4 blo = {__builtin_bit_cast(float, b[0] << 16), __builtin_bit_cast(float, b[0] & 0xFFFF0000u),
                               __builtin_bit_cast(float, b[1] << 16), __builtin_bit_cast(float, b[1] & 0xFFFF0000u)};
          const floatx4 bhi = {__builtin_bit_cast(float, b[2] << 16), __builtin_bit_cast(float, b[2] & 0xFFFF0000u),
                               __builtin_bit_cast(float, b[3] << 16), __builtin_bit_cast(float, b[3] & 0xFFFF0000u)};
          float sc = 1.0f;
          if (bscale) {
            const uint32_t r = (uint32_t)(32 * TMA * wm + 32 * i + 8 * q) + opaque_v((uint32_t)(lane >> 3));
            sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                               make_rsrc(bscale, (uint32_t)rows * 4u), r * 4u, 0, 0));
          }
          lo = lo + blo * sc;
          hi = hi + bhi * sc;
        }
      }
      if constexpr (OUT_F32) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, lo), rs, voff, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hi), rs, voff + 16, 0, 0);
      } else {
        u32x4 o = {pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                   pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
        __builtin_amdgcn_raw_buffer_store_b128(o, rs, voff, 0, 0);
      }
      // one slab row group at a time (hoisting the prior-output loads of
      // all four would need 32 more registers)
      if constexpr (SCALED) __builtin_amdgcn_sched_barrier(0);
    }
    // the next block row rewrites the slab: wait for this row's reads
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  }
}

// The SiLU-mul epilogue of a gate/up tile: waves 0, 1 (mod 4) hold the gate
// columns 64 wn .. of the tile's 128 activation columns and waves 2, 3 the
// matching up columns, so the two halves meet in LDS.  Per block row every
// wave writes its 32 x 64 fp32 slab (as store_tile_lds does) and all waves
// meet; then the gate wave and its up partner (wave + 2) share the slab
// pair, the gate wave taking slab rows 0..15 and the up wave rows 16..31:
// each lane reads 8 consecutive gate values and the 8 matching up values,
// writes silu(g) * u = g * rcp(1 + exp(-g)) * u in fp32, rounded once to the
// output type, and all waves meet again before the slabs are rewritten.
// `slabs` is the idle stage-buffer area; each wave's slab is 16 KB apart.
template <int TMA, bool OUT_F32>
__device__ __forceinline__ void store_tile_silu(uint8_t* cbase, uint32_t ldc_bytes, int rows, int cols,
                                                int wave, int wm, int wn, int lane,
                                                const floatx16 (&acc)[TM][TN], uint8_t* slabs) {
  constexpr uint32_t esz = OUT_F32 ? 4 : 2;
  constexpr uint32_t kSlabStride = STAGE_BYTES / 2;
  const uint32_t nrec = (uint32_t)(rows - 1) * ldc_bytes + (uint32_t)cols * esz;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(cbase, nrec);
  uint8_t* own = slabs + wave * kSlabStride;
  const bool gate_wave = wn < 2;
  const uint8_t* gslab = slabs + (gate_wave ? wave : wave - 2) * kSlabStride;
  const uint8_t* uslab = gslab + 2 * kSlabStride;
  const int q0 = gate_wave ? 0 : 2;                // slab row groups this wave combines
  const uint32_t wslab = opaque_v((uint32_t)((lane & 31) * kSlabPitch + 16 * (lane >> 5)));
  const uint32_t rslab = opaque_v((uint32_t)((lane >> 3) * kSlabPitch + 32 * (lane & 7)));
  const int gcol = 64 * (wn & 1) + 8 * (lane & 7);   // activation column
  const bool col_ok = gcol < cols;
  const uint32_t gbase = col_ok ? opaque_v((uint32_t)(32 * TMA * wm + (lane >> 3)) * ldc_bytes +
                                           (uint32_t)gcol * esz)
                                : kOutOfRange;
#pragma unroll
  for (int i = 0; i < TMA; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        floatx4 v = {acc[i][j][4 * rr + 0], acc[i][j][4 * rr + 1], acc[i][j][4 * rr + 2], acc[i][j][4 * rr + 3]};
        *reinterpret_cast<floatx4*>(own + wslab + 4 * (32 * j + 8 * rr)) = v;
      }
    lds_barrier();
    {
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int q = q0 + qq;
        float g[8], u[8], o[8];
        *reinterpret_cast<floatx4*>(&g[0]) = *reinterpret_cast<const floatx4*>(gslab + rslab + 8 * q * kSlabPitch);
        *reinterpret_cast<floatx4*>(&g[4]) = *reinterpret_cast<const floatx4*>(gslab + rslab + 8 * q * kSlabPitch + 16);
        *reinterpret_cast<floatx4*>(&u[0]) = *reinterpret_cast<const floatx4*>(uslab + rslab + 8 * q * kSlabPitch);
        *reinterpret_cast<floatx4*>(&u[4]) = *reinterpret_cast<const floatx4*>(uslab + rslab + 8 * q * kSlabPitch + 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = g[e] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[e])) * u[e];
        const uint32_t voff = gbase + (uint32_t)(32 * i + 8 * q) * ldc_bytes;
        if constexpr (OUT_F32) {
          const floatx4 lo = {o[0], o[1], o[2], o[3]};
          const floatx4 hi = {o[4], o[5], o[6], o[7]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, lo), rs, voff, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hi), rs, voff + 16, 0, 0);
        } else {
          const u32x4 w = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                           pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
          __builtin_amdgcn_raw_buffer_store_b128(w, rs, voff, 0, 0);
        }
      }
    }
    // every slab is rewritten by the next block row
    lds_barrier();
  }
}

// ---- group decode (prologue) ---------------------------------------------------

// Block-wide inclusive scan of one value per thread (sum or max).
template <bool MAX, typename T>
__device__ __forceinline__ T block_scan_incl(T v, T* scratch, int tid) {
  scratch[tid] = v;
  __syncthreads();
#pragma unroll
  for (int d = 1; d < NT; d <<= 1) {
    T o = tid >= d ? scratch[tid - d] : T(0);
    __syncthreads();
    if (tid >= d) v = MAX ? (v > o ? v : o) : v + o;
    scratch[tid] = v;
    __syncthreads();
  }
  return v;
}

// wgrad takes its experts longest first when there are at most this many
// (the ordering costs each workgroup E^2 / 512 comparisons).
constexpr int kOrderMaxGroups = 512;

// First row of group g within its row range (the ragged layout's groups
// follow one another; a masked group's rows start at 0 of its block).
template <int MODE>
__device__ __forceinline__ int group_start(const int32_t* s_end, int g) {
  return is_masked(MODE) || g == 0 ? 0 : s_end[g - 1];
}

// A group's last row tile runs at half height when it holds BM/2 rows or
// fewer; every other row tile runs at full height.
__device__ __forceinline__ int half_tiles(int rows) {
  const int r = rows % BM;
  return r != 0 && r <= BM / 2 ? 1 : 0;
}

// Fills s_end with the clamped end row of every group and, unless a wgrad
// mode, s_pref[0..E] with the exclusive prefix of the groups' full-height
// row-tile counts and s_half[0..E] with that of their half-height last
// tiles (0 or 1 per group).
template <int MODE>
__device__ void decode_groups(const Params& p, int32_t* s_end, int32_t* s_pref, int32_t* s_half,
                              int64_t* scratch, int tid) {
  const int E = p.num_groups;
  const int per = (E + NT - 1) / NT;
  const int g0 = tid * per;
  const int g1 = g0 + per < E ? g0 + per : E;
  if constexpr (is_masked(MODE)) {
    for (int g = g0; g < g1; ++g) {
      int a = p.groups[g];
      a = a < 0 ? 0 : a;
      a = a > p.m ? (int)p.m : a;
      s_end[g] = a;
    }
  } else {
    // end(g) = min(max(0, offs[0..g]), M): a prefix max.
    int run = 0;
    for (int g = g0; g < g1; ++g) {
      int o = p.groups[g];
      run = o > run ? o : run;
      s_end[g] = run;
    }
    block_scan_incl<true, int64_t>(run, scratch, tid);
    const int before = tid > 0 ? (int)scratch[tid - 1] : 0;
    __syncthreads();
    const int mcap = (int)p.m;
    for (int g = g0; g < g1; ++g) {
      int e = s_end[g] > before ? s_end[g] : before;
      s_end[g] = e < mcap ? e : mcap;
    }
  }
  __syncthreads();
  if constexpr (!is_wgrad(MODE)) {
    // (full, half) counts packed as full + half * 2^32: both stay below 2^31
    int64_t local = 0;
    for (int g = g0; g < g1; ++g) {
      const int rows = s_end[g] - group_start<MODE>(s_end, g);
      const int h = half_tiles(rows);
      local += (int64_t)((rows + BM - 1) / BM - h) + ((int64_t)h << 32);
    }
    const int64_t incl = block_scan_incl<false, int64_t>(local, scratch, tid);
    int full = (int)((incl - local) & 0xffffffff);
    int half = (int)((incl - local) >> 32);
    for (int g = g0; g < g1; ++g) {
      s_pref[g] = full;
      s_half[g] = half;
      const int rows = s_end[g] - group_start<MODE>(s_end, g);
      const int h = half_tiles(rows);
      full += (rows + BM - 1) / BM - h;
      half += h;
    }
    if (tid == NT - 1) {
      s_pref[E] = (int)(incl & 0xffffffff);
      s_half[E] = (int)(incl >> 32);
    }
    __syncthreads();
  } else if (E <= kOrderMaxGroups) {
    // wgrad: a wgrad tile lasts as many stages as its expert has 32-row
    // blocks, and every expert has the same number of tiles.  Take the
    // experts longest first -- by a quarter-octave class of their stage
    // count, ties by index -- so that the persistent loop ends on short tiles
    // (and, with rounds alternating direction, every workgroup gets about the
    // same work).  The order is a function of the offsets alone, identical
    // in every workgroup: key k(g) = class * 4096 + 4095 - g is unique, and
    // an expert's rank is the number of larger keys.  s_half holds the keys,
    // s_pref[rank] the expert.
    for (int g = tid; g < E; g += NT) {
      const int stages = (s_end[g] - group_start<MODE>(s_end, g) + 31) >> 5;
      const int cls = (int)(4.0f * __log2f((float)(stages + 1)));
      s_half[g] = cls * 4096 + (4095 - g);
    }
    __syncthreads();
    for (int g = tid; g < E; g += NT) {
      const int key = s_half[g];
      int rank = 0;
      for (int h = 0; h < E; ++h) rank += s_half[h] > key ? 1 : 0;
      s_pref[rank] = g;
    }
    __syncthreads();
  }
}

// Largest g in [0, E) with pref[g] <= t (pref is a non-decreasing
// exclusive prefix, pref[0] = 0 <= t < pref[E]).  That group's count is
// non-zero: pref[g] <= t < pref[g + 1].
__device__ __forceinline__ int find_group(const int32_t* pref, int E, int t) {
  int lo = 0, hi = E;          // invariant: pref[lo] <= t < pref[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (pref[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// ---- tile order -------------------------------------------------------------------

// Workgroups are dealt to the 8 XCDs (each with its own L2) round-robin:
// workgroup b runs on XCD b mod 8.  Within each round of gridDim.x tiles,
// workgroup b takes position (b mod 8) (G / 8) + b / 8, so each XCD works on
// a contiguous run of the order below.  The last, partial round keeps the
// plain order (any bijection works there).
// snake: odd rounds take the positions in reverse (wgrad with its experts
// longest first, where consecutive rounds then even out).
__device__ __forceinline__ int64_t xcd_tile(int64_t t, int64_t total, bool snake) {
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int64_t round0 = t - b;
  if ((G & 7) != 0 || round0 + G > total) return t;
  int64_t pos = (int64_t)(b & 7) * (G >> 3) + (b >> 3);
  if (snake && ((round0 / G) & 1)) pos = G - 1 - pos;
  return round0 + pos;
}

// Order of an rows x cols grid of tiles: column strips of (up to) 8 tiles,
// each strip walked row by row, so a run of 32 consecutive tiles is a block
// of 4 tile rows x 8 tile columns (4 A panels and 8 B panels shared within
// one XCD).  Returns (row, col) of linear index u.
constexpr int kStrip = 8;
__device__ __forceinline__ void strip_order(int64_t u, int64_t rows, int cols, int64_t& r, int& c) {
  const int bw = cols < kStrip ? cols : kStrip;
  const int full = cols / bw;                    // strips of width bw
  const int64_t per = rows * bw;
  if (u < (int64_t)full * per) {
    const int s = (int)(u / per);
    const int64_t w = u - (int64_t)s * per;
    r = w / bw;
    c = s * bw + (int)(w - r * bw);
  } else {
    const int rem = cols - full * bw;            // last, narrower strip
    const int64_t w = u - (int64_t)full * per;
    r = w / rem;
    c = full * bw + (int)(w - r * rem);
  }
}

// ---- the kernel ------------------------------------------------------------------

// One output tile: its operands and output window.
struct Tile {
  Operand A, B;
  uint8_t* cbase;       // output element (first row, first column) of the tile
  uint32_t ldc_bytes;   // output row pitch
  int rows, cols;       // valid output rows / columns of the tile
  const uint8_t* sa;    // fp8: the tile's packed X scales (k-block 0)
  const uint8_t* sb;    // fp8: the tile's packed W scales
  const uint16_t* bias;   // the expert's bias at the tile's first column, or null
  const float* bscale;    // the bias factor of the tile's first row, or null
};


// STAGED_F32: fp32 output through the LDS epilogue even when unscaled (the
// host picks it for wgrad on short experts; see launch()).  WIDE (wgrad
// only): an expert's rows may span 4 GB or more of X or dY, so the load
// ranges are capped per stage (see dma_ctx_grp); the host picks it from m.
template <int MODE, bool OUT_F32, bool STAGED_F32 = false, bool WIDE = false>
__global__ __launch_bounds__(NT, 1) void grouped_gemm_kernel(Params p) {
  static_assert(!WIDE || is_wgrad(MODE), "only wgrad reads an operand down a data-dependent span");
  constexpr bool A_STRIDED = is_wgrad(MODE);
  constexpr bool B_STRIDED = !is_dgrad(MODE) && !is_fp8(MODE);
  // Main loops: the bf16 row passes ping-pong with A in the pair layout,
  // wgrad ping-pongs with one stage per slot for both operands, the fp8
  // forward runs the row passes' schedule on bytes (mainloop8_pp).
  constexpr bool PP_PAIR = !is_wgrad(MODE) && !is_fp8(MODE);

  // LDS: NSTAGE stage buffers of 32 KB (A tile, then B tile); fp8: two
  // k-blocks of scales.
  __shared__ __attribute__((aligned(16))) uint8_t smem[NSTAGE * STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_sc[is_fp8(MODE) ? 2 * kScaleSlot : 16];
  __shared__ int32_t s_end[GG_MAX_GROUPS_DEV];
  __shared__ int32_t s_pref[GG_MAX_GROUPS_DEV + 1];
  __shared__ int32_t s_half[GG_MAX_GROUPS_DEV + 1];
  __shared__ int64_t s_scan[NT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);     // wave index, held in a scalar register
  const int wm = wave >> 2;
  const int wn = wave & 3;
  const int E = p.num_groups;

  decode_groups<MODE>(p, s_end, s_pref, s_half, s_scan, tid);

  // Output tile grid.  A SiLU tile writes 128 activation columns from a
  // 256-column panel: 128 gate columns and the 128 matching up columns.
  constexpr int kOutCols = is_silu(MODE) ? BN / 2 : BN;
  const int64_t out_cols = is_dgrad(MODE) ? p.k : is_silu(MODE) ? p.n / 2 : p.n;
  const int col_tiles = (int)((out_cols + kOutCols - 1) / kOutCols);
  // Non-wgrad tiles come in two phases: every full-height row tile, then
  // the half-height last tiles.  Tiles of one phase take the same time, so
  // the workgroups of an XCD stay in step and share their panels in L2.
  int64_t total;
  int64_t full_tiles = 0;
  int row_tiles_w = 0;
  if constexpr (is_wgrad(MODE)) {
    row_tiles_w = (int)((p.k + BM - 1) / BM);
    total = (int64_t)E * row_tiles_w * col_tiles;
  } else {
    full_tiles = (int64_t)uniform(s_pref[E]) * col_tiles;
    total = full_tiles + (int64_t)uniform(s_half[E]) * col_tiles;
  }


  constexpr uint32_t esz = OUT_F32 ? 4 : 2;
  const uint8_t* pa = reinterpret_cast<const uint8_t*>(p.a);
  const uint8_t* pb = reinterpret_cast<const uint8_t*>(p.b);
  uint8_t* pc = reinterpret_cast<uint8_t*>(p.c);
  // A in the pair layout for the row passes (bf16 and fp8), one stage per slot for wgrad
  constexpr bool A_PAIRED = !is_wgrad(MODE);
  const FragAddr faa = A_PAIRED ? frag_addr_pair(128 * wm, lane) : frag_addr<A_STRIDED>(128 * wm, lane);
  // half-height tiles
  const FragAddr faa_half = A_PAIRED ? frag_addr_pair(64 * wm, lane) : frag_addr<A_STRIDED>(64 * wm, lane);
  const FragAddr fab = frag_addr<B_STRIDED>(64 * wn, lane);
  uint8_t* const sa0 = smem;
  uint8_t* const sa1 = smem + STAGE_BYTES;
  uint8_t* const sa2 = smem + 2 * STAGE_BYTES;
  uint8_t* const sa3 = smem + 3 * STAGE_BYTES;

  // Decode tile t (linear index over the output tile grid) into its
  // operand descriptions and output window.
  // wgrad experts longest first (see decode_groups)
  const bool ordered = is_wgrad(MODE) && E <= kOrderMaxGroups;
  auto decode_tile = [&](int64_t t, Tile& T) __attribute__((always_inline)) {
    const int64_t u = xcd_tile(t, total, ordered);
    int ct;
    int64_t rt_all;
    if constexpr (is_wgrad(MODE)) {
      // per expert: a row_tiles_w x col_tiles grid in strip order
      const int64_t per_g = (int64_t)row_tiles_w * col_tiles;
      const int64_t gq = u / per_g;             // position of the expert in the order
      int64_t rr;
      strip_order(u - gq * per_g, row_tiles_w, col_tiles, rr, ct);
      const int64_t gx = ordered ? (int64_t)uniform(s_pref[gq]) : gq;
      rt_all = gx * row_tiles_w + rr;
    } else if (u < full_tiles) {
      strip_order(u, full_tiles / col_tiles, col_tiles, rt_all, ct);
    } else {
      strip_order(u - full_tiles, (total - full_tiles) / col_tiles, col_tiles, rt_all, ct);
    }
    const int col0 = ct * kOutCols;
    Operand& A = T.A;
    Operand& B = T.B;
    A.split = 0;
    B.split = 0;
    T.sa = nullptr;
    T.sb = nullptr;
    T.bias = nullptr;
    T.bscale = nullptr;
    if constexpr (is_wgrad(MODE)) {
      const int g = (int)(rt_all / row_tiles_w);
      const int rt = (int)(rt_all % row_tiles_w);
      const int row0 = rt * BM;                 // first k index of the tile
      const int s = uniform(group_start<MODE>(s_end, g)), e = uniform(s_end[g]);
      // first memory row of the expert's rows (masked: expert g's block)
      const int64_t srow = (is_masked(MODE) ? (int64_t)g * p.m : 0) + s;
      // A(row kk, red i) = X[srow + i, row0 + kk]
      A.origin = pa + 2 * (srow * p.k + row0);
      A.ld_bytes = (uint32_t)(2 * p.k);
      A.rows = (int)(p.k - row0 < BM ? p.k - row0 : BM);
      A.red = e - s;
      A.row_tail = (uint32_t)(2 * (p.k - row0));
      // B(row n, red i) = dY[srow + i, col0 + n]
      B.origin = pb + 2 * (srow * p.n + col0);
      B.ld_bytes = (uint32_t)(2 * p.n);
      B.rows = (int)(p.n - col0 < BN ? p.n - col0 : BN);
      B.red = e - s;
      B.row_tail = (uint32_t)(2 * (p.n - col0));
      T.ldc_bytes = (uint32_t)(esz * p.n);
      T.cbase = pc + esz * ((int64_t)g * p.k * p.n + (int64_t)row0 * p.n + col0);
      T.rows = A.rows;
      T.cols = B.rows;
    } else {
      // full phase: row tile rt_all - s_pref[g] of group g; half phase:
      // the last row tile of group g
      const bool in_full = u < full_tiles;
      const int g = uniform(find_group(in_full ? s_pref : s_half, E, (int)rt_all));
      const int s = uniform(group_start<MODE>(s_end, g)), e = uniform(s_end[g]);
      const int rt = in_full ? (int)rt_all - uniform(s_pref[g]) : (e - s - 1) / BM;
      const int row0 = s + rt * BM;             // first expert row of the tile
      const int rows = (e - row0) < BM ? (e - row0) : BM;
      const int64_t arow = is_masked(MODE) ? (int64_t)g * p.m + row0 : (int64_t)row0;
      if constexpr (is_fp8(MODE)) {
        // A(row i, red kk) = X[arow + i, kk];  B(row n, red kk) = W[g, col0 + n, kk]
        // (one byte per value)
        A.origin = pa + arow * p.k;
        A.ld_bytes = (uint32_t)p.k;
        A.rows = rows;
        A.red = (int)p.k;
        A.row_tail = 0;
        B.origin = pb + ((int64_t)g * p.n + col0) * p.k;
        B.ld_bytes = (uint32_t)p.k;
        B.rows = (int)(p.n - col0 < BN ? p.n - col0 : BN);
        B.red = (int)p.k;
        B.row_tail = 0;
        T.ldc_bytes = (uint32_t)(esz * p.n);
        T.cbase = pc + esz * (arow * p.n + col0);
        // packed scale tiles: X row tile (experts in order), W column tile
        const int64_t kblocks = p.k / 128;
        const int64_t xtile = is_masked(MODE) ? (int64_t)g * ((p.m + BM - 1) / BM) + rt
                                              : (int64_t)uniform(s_pref[g]) + uniform(s_half[g]) + rt;
        T.sa = p.sa + xtile * kblocks * 256;
        T.sb = p.sb + ((int64_t)g * ((p.n + BN - 1) / BN) + ct) * kblocks * 256;
      } else if constexpr (is_dgrad(MODE)) {
        // A(row i, red j) = dY[arow + i, j];  B(row kk, red j) = W[g, col0 + kk, j]
        A.origin = pa + 2 * (arow * p.n);
        A.ld_bytes = (uint32_t)(2 * p.n);
        A.rows = rows;
        A.red = (int)p.n;
        A.row_tail = 0;
        B.origin = pb + 2 * ((int64_t)g * p.k * p.n + (int64_t)col0 * p.n);
        B.ld_bytes = (uint32_t)(2 * p.n);
        B.rows = (int)(p.k - col0 < BN ? p.k - col0 : BN);
        B.red = (int)p.n;
        B.row_tail = 0;
        T.ldc_bytes = (uint32_t)(esz * p.k);
        T.cbase = pc + esz * (arow * p.k + col0);
      } else {
        // A(row i, red kk) = X[arow + i, kk];  B(row n, red kk) = W[g, kk, col0 + n]
        A.origin = pa + 2 * (arow * p.k);
        A.ld_bytes = (uint32_t)(2 * p.k);
        A.rows = rows;
        A.red = (int)p.k;
        A.row_tail = 0;
        B.origin = pb + 2 * ((int64_t)g * p.k * p.n + col0);
        B.ld_bytes = (uint32_t)(2 * p.n);
        B.rows = (int)(p.n - col0 < BN ? p.n - col0 : BN);
        B.red = (int)p.k;
        B.row_tail = (uint32_t)(2 * (p.n - col0));
        T.ldc_bytes = (uint32_t)(esz * p.n);
        T.cbase = pc + esz * (arow * p.n + col0);
        if constexpr (is_silu(MODE)) {
          // gate columns col0.. in tile rows 0..127, up columns I + col0..
          // in tile rows 128..255; the output is the I-wide activation
          const int64_t half_n = p.n / 2;
          B.split = (uint32_t)(2 * (half_n - BN / 2));
          B.rows = (int)(half_n - col0 < kOutCols ? half_n - col0 : kOutCols);
          T.ldc_bytes = (uint32_t)(esz * half_n);
          T.cbase = pc + esz * (arow * half_n + col0);
        }
      }
      T.rows = rows;
      T.cols = B.rows;
      if constexpr (has_bias(MODE)) {
        if (p.bias) {
          T.bias = p.bias + (int64_t)g * p.n + col0;
          T.bscale = p.bias_scale ? p.bias_scale + arow : nullptr;
        }
      }
    }
  };
  auto issue_prologue = [&](const Tile& T) __attribute__((always_inline)) {
    if (T.A.red > 0) {
      if constexpr (is_fp8(MODE))
        prologue_loads8_pp(sa0, sa1, sa2, sa0 + OP_BYTES, sa1 + OP_BYTES, sa2 + OP_BYTES, s_sc, T.A.origin,
                           T.B.origin, T.sa, T.sb, (uint32_t)(p.k / 128 * 256), T.A, T.B, tid, wave);
      else if constexpr (PP_PAIR)
        prologue_loads_pp_pair<B_STRIDED>(sa0, sa1, sa2, sa3, sa0 + OP_BYTES, sa1 + OP_BYTES, sa2 + OP_BYTES,
                                          T.A.origin, T.B.origin, T.A, T.B, tid, wave);
      else
        prologue_loads_pp<A_STRIDED, B_STRIDED, WIDE>(smem, smem + STAGE_BYTES, smem + 2 * STAGE_BYTES,
                                                      smem + 3 * STAGE_BYTES, T.A.origin, T.B.origin, T.A,
                                                      T.B, tid, wave);
    }
  };

  if ((int64_t)blockIdx.x >= total) return;
  // Decodes below use an index clamped into the grid, so every Tile is
  // assigned on every path (it stays in scalar registers).
  const int64_t last = total - 1;
  Tile cur;
  decode_tile(blockIdx.x, cur);
  issue_prologue(cur);
  int prev_stores = 0;    // fp32 stores issued after the current tile's prologue loads
  // The scaled form (alpha != 1 or beta != 0) goes through the LDS epilogue
  // for both output types.
  const bool scaled = p.alpha != 1.0f || p.beta != 0.0f || p.bias != nullptr;
  for (int64_t t = blockIdx.x; t < total; t += gridDim.x) {
    floatx16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // An expert's last tile with 128 rows or fewer runs at half height:
    // each wave computes 64 x 64, skipping the MFMAs of empty rows.
    const bool half = !is_wgrad(MODE) && cur.rows <= BM / 2;
    // fp32 tiles after the first start with the previous tile's stores
    // still in flight behind their prologue loads
    if constexpr (is_fp8(MODE)) {
      const uint32_t sc_bytes = (uint32_t)(p.k / 128 * 256);
      if (half)
        mainloop8_pp<2>(sa0, sa1, sa2, sa3, sa0 + OP_BYTES, sa1 + OP_BYTES, sa2 + OP_BYTES, sa3 + OP_BYTES,
                        s_sc, cur.A.origin, cur.B.origin, cur.sa, cur.sb, sc_bytes, cur.A, cur.B, tid, wave, wm,
                        wn, 0, faa_half, fab, acc);
      else
        mainloop8_pp<TM>(sa0, sa1, sa2, sa3, sa0 + OP_BYTES, sa1 + OP_BYTES, sa2 + OP_BYTES, sa3 + OP_BYTES,
                         s_sc, cur.A.origin, cur.B.origin, cur.sa, cur.sb, sc_bytes, cur.A, cur.B, tid, wave, wm,
                         wn, wm, faa, fab, acc);
    } else if constexpr (PP_PAIR) {
      // the wave's A rows: 128 wm.. (full height, region wm) or 64 wm.. (half, region 0)
      if (half)
        mainloop_pp_pair<B_STRIDED, 2>(sa0, sa1, sa2, sa3, sa0 + OP_BYTES, sa1 + OP_BYTES, sa2 + OP_BYTES,
                                       sa3 + OP_BYTES, cur.A.origin, cur.B.origin, cur.A, cur.B, tid, wave, 0,
                                       faa_half, fab, acc, prev_stores);
      else
        mainloop_pp_pair<B_STRIDED, TM>(sa0, sa1, sa2, sa3, sa0 + OP_BYTES, sa1 + OP_BYTES, sa2 + OP_BYTES,
                                        sa3 + OP_BYTES, cur.A.origin, cur.B.origin, cur.A, cur.B, tid, wave, wm,
                                        faa, fab, acc, prev_stores);
    } else {
      if (half)
        mainloop_pp<A_STRIDED, B_STRIDED, 2, WIDE>(smem, smem + STAGE_BYTES, smem + 2 * STAGE_BYTES,
                                                   smem + 3 * STAGE_BYTES, cur.A.origin, cur.B.origin, cur.A,
                                                   cur.B, tid, wave, faa_half, fab, acc, prev_stores);
      else
        mainloop_pp<A_STRIDED, B_STRIDED, TM, WIDE>(smem, smem + STAGE_BYTES, smem + 2 * STAGE_BYTES,
                                                    smem + 3 * STAGE_BYTES, cur.A.origin, cur.B.origin, cur.A,
                                                    cur.B, tid, wave, faa, fab, acc, prev_stores);
    }
    const int64_t tn = t + gridDim.x;
    if (OUT_F32 && !STAGED_F32 && !scaled && !is_silu(MODE) && !is_fp8(MODE)) {
      // Every wave is done reading this tile's stages: issue the next
      // tile's prologue loads first, then this tile's stores, so the
      // stores drain while those loads are in flight.  (Loads of stages
      // past this tile's end may still be landing zeros: they complete
      // before the next tile's, in issue order.)
      lds_barrier();
      Tile nxt;
      decode_tile(tn < total ? tn : last, nxt);
      if (tn < total) issue_prologue(nxt);
      if (half) {
        store_tile_f32<2>(cur.cbase, cur.ldc_bytes, cur.rows, cur.cols, wm, wn, lane, acc);
        prev_stores = stores_f32<2>();
      } else {
        store_tile_f32<TM>(cur.cbase, cur.ldc_bytes, cur.rows, cur.cols, wm, wn, lane, acc);
        prev_stores = stores_f32<TM>();
      }
      cur = nxt;
    } else {
      // loads of stages past the end may still be landing (zeros), and
      // other waves may still read the last stage: settle before the LDS
      // is reused as the epilogue's staging area
      stage_barrier();
      // each wave stages through its own 16 KB of the (idle) stage buffers
      uint8_t* slab = smem + wave * (STAGE_BYTES / 2);
      if constexpr (is_silu(MODE)) {
        if (half)
          store_tile_silu<2, OUT_F32>(cur.cbase, cur.ldc_bytes, cur.rows, cur.cols, wave, wm, wn, lane,
                                      acc, smem);
        else
          store_tile_silu<TM, OUT_F32>(cur.cbase, cur.ldc_bytes, cur.rows, cur.cols, wave, wm, wn, lane,
                                       acc, smem);
      } else if (scaled) {
        if (half)
          store_tile_lds<2, OUT_F32, true>(cur.cbase, cur.ldc_bytes, cur.rows, cur.cols, wm, wn, lane,
                                           acc, slab, p.alpha, p.beta, cur.bias, cur.bscale);
        else
          store_tile_lds<TM, OUT_F32, true>(cur.cbase, cur.ldc_bytes, cur.rows, cur.cols, wm, wn, lane,
                                            acc, slab, p.alpha, p.beta, cur.bias, cur.bscale);
      } else if constexpr (!OUT_F32 || is_fp8(MODE) || STAGED_F32) {
        if (half)
          store_tile_lds<2, OUT_F32, false>(cur.cbase, cur.ldc_bytes, cur.rows, cur.cols, wm, wn, lane,
                                            acc, slab, 1.0f, 0.0f);
        else
          store_tile_lds<TM, OUT_F32, false>(cur.cbase, cur.ldc_bytes, cur.rows, cur.cols, wm, wn, lane,
                                             acc, slab, 1.0f, 0.0f);
      }
      prev_stores = 0;
      // the next tile's first loads overwrite these arrays
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __syncthreads();
      decode_tile(tn < total ? tn : last, cur);
      if (tn < total) issue_prologue(cur);
    }
  }
}

// ---- host-side launchers -------------------------------------------------------

template <int MODE, bool OUT_F32, bool STAGED_F32 = false, bool WIDE = false>
static hipError_t launch_one(const Params& p, int grid, hipStream_t stream) {
  return launch_kernel(grouped_gemm_kernel<MODE, OUT_F32, STAGED_F32, WIDE>, dim3(grid), dim3(NT), stream, p);
}

// Unscaled fp32 wgrad tiles store straight from the accumulators, with the
// next tile's first loads issued ahead of the stores.  When experts are short
// (fewer rows per expert on average than this), tiles are bound by those
// stores, and they go out faster staged through LDS as whole rows (measured:
// Qwen3 gate/up and DSV3-class wgrad 7-9 % faster; GLM-up's long experts 2-3 %
// slower staged).
constexpr int64_t kStagedF32Rows = 2048;

template <int MODE>
static hipError_t launch_mode(const Params& p, bool out_f32, int grid, hipStream_t stream) {
  return out_f32 ? launch_one<MODE, true>(p, grid, stream) : launch_one<MODE, false>(p, grid, stream);
}

// wgrad reads X and dY down each expert's rows, one buffer range per stage
// running to the expert's last row.  When an expert could span 4 GB of
// either (bounded by all m rows, or max_m), the kernel caps those ranges.
template <int MODE>
static hipError_t launch_wgrad(const Params& p, bool out_f32, bool staged, int grid, hipStream_t stream) {
  const int64_t widest = 2 * (p.k > p.n ? p.k : p.n);
  if (p.m * widest < (int64_t(1) << 32)) {
    if (staged) return launch_one<MODE, true, true>(p, grid, stream);
    return launch_mode<MODE>(p, out_f32, grid, stream);
  }
  if (staged) return launch_one<MODE, true, true, true>(p, grid, stream);
  return out_f32 ? launch_one<MODE, true, false, true>(p, grid, stream)
                 : launch_one<MODE, false, false, true>(p, grid, stream);
}

// Upper bound on the number of output tiles, from host-known sizes only
// (the device knows the exact count).  Each expert adds at most one partial
// row tile beyond ceil(rows / BM).
static int64_t max_tiles(int mode, int64_t m, int64_t k, int64_t n, int64_t E) {
  if (is_wgrad(mode)) return E * ((k + BM - 1) / BM) * ((n + BN - 1) / BN);
  if (is_silu(mode)) {
    const int64_t ct = (n / 2 + BN / 2 - 1) / (BN / 2);
    if (is_masked(mode)) return E * ((m + BM - 1) / BM) * ct;
    return ((m + BM - 1) / BM + E) * ct;
  }
  const int64_t cols = is_dgrad(mode) ? k : n;
  const int64_t ct = (cols + BN - 1) / BN;
  if (is_masked(mode)) return E * ((m + BM - 1) / BM) * ct;
  return ((m + BM - 1) / BM + E) * ct;
}

hipError_t launch(int mode, const void* a, const void* b, const int32_t* groups, void* c,
                  bool out_f32, int64_t m, int64_t k, int64_t n, int32_t num_groups,
                  float alpha, float beta, const void* bias, const float* bias_scale, int num_cus,
                  hipStream_t stream) {
  Params p;
  p.a = static_cast<const uint16_t*>(a);
  p.b = static_cast<const uint16_t*>(b);
  p.groups = groups;
  p.c = c;
  p.m = m;
  p.k = k;
  p.n = n;
  p.num_groups = num_groups;
  p.alpha = alpha;
  p.beta = beta;
  p.sa = nullptr;
  p.sb = nullptr;
  p.bias = static_cast<const uint16_t*>(bias);
  p.bias_scale = bias_scale;
  const int64_t tiles = max_tiles(mode, m, k, n, num_groups);
  if (tiles <= 0) return hipSuccess;
  const int grid = (int)(tiles < num_cus ? tiles : num_cus);
  switch (mode) {
    case FWD: return launch_mode<FWD>(p, out_f32, grid, stream);
    case DGRAD: return launch_mode<DGRAD>(p, out_f32, grid, stream);
    case WGRAD:
      return launch_wgrad<WGRAD>(p, out_f32, out_f32 && alpha == 1.0f && beta == 0.0f &&
                                                 m / num_groups < kStagedF32Rows, grid, stream);
    case MASKED: return launch_mode<MASKED>(p, out_f32, grid, stream);
    case MASKED_DGRAD: return launch_mode<MASKED_DGRAD>(p, out_f32, grid, stream);
    case MASKED_WGRAD:
      return launch_wgrad<MASKED_WGRAD>(p, out_f32, out_f32 && alpha == 1.0f && beta == 0.0f &&
                                                       m < kStagedF32Rows, grid, stream);
    case FWD_SILU: return launch_mode<FWD_SILU>(p, out_f32, grid, stream);
    case MASKED_SILU: return launch_mode<MASKED_SILU>(p, out_f32, grid, stream);
  }
  return hipErrorInvalidValue;
}


hipError_t launch_fp8(bool masked, const void* x, const void* sx, const void* w, const void* sw,
                      const int32_t* groups, void* c, bool out_f32, int64_t m, int64_t k, int64_t n,
                      int32_t num_groups, int num_cus, hipStream_t stream) {
  Params p;
  p.a = static_cast<const uint16_t*>(x);
  p.b = static_cast<const uint16_t*>(w);
  p.groups = groups;
  p.c = c;
  p.m = m;
  p.k = k;
  p.n = n;
  p.num_groups = num_groups;
  p.alpha = 1.0f;
  p.beta = 0.0f;
  p.sa = static_cast<const uint8_t*>(sx);
  p.sb = static_cast<const uint8_t*>(sw);
  p.bias = nullptr;
  p.bias_scale = nullptr;
  const int mode = masked ? FP8_MASKED : FP8;
  const int64_t tiles = max_tiles(mode, m, k, n, num_groups);
  if (tiles <= 0) return hipSuccess;
  const int grid = (int)(tiles < num_cus ? tiles : num_cus);
  return masked ? launch_mode<FP8_MASKED>(p, out_f32, grid, stream)
                : launch_mode<FP8>(p, out_f32, grid, stream);
}

}  // namespace gg
