// gg_kernels.hip -- persistent bf16 grouped-GEMM kernels for gfx950 (CDNA4).
//
// One kernel template serves the four passes of the grouped GEMM (forward,
// dgrad, wgrad and the masked forward; see include/gg.h for the operations
// and the passages that define them).  Each pass is the same tile engine fed
// by a different operand description:
//
//   pass     out tile rows x cols      reduction   A operand           B operand
//   forward  expert rows  x n          k           X   (red-contig)    W[g] (red-strided)
//   dgrad    expert rows  x k          n           dY  (red-contig)    W[g] (red-contig)
//   wgrad    k            x n          expert rows X   (red-strided)   dY   (red-strided)
//   masked   active rows  x n          k           X[e] (red-contig)   W[e] (red-strided)
//
// "red-contig" means the reduction index is the contiguous one in memory;
// "red-strided" means the tile's row index is.  Both land in LDS in one
// layout -- tile row r holds its 64 reduction values contiguously (128 B),
// the 16-byte chunk c stored at chunk position c ^ (r & 7) so that the eight
// lanes served together by an LDS access touch eight different chunks.
// Red-strided operands are transposed 8 x 8 in registers on their way into
// LDS (32 byte permutes per thread per stage).
//
// Work decomposition (no host sync, no workspace): the launch has one
// workgroup per compute unit.  Each workgroup decodes the device-side end
// offsets (or masked_m) into LDS -- clamped ends by a prefix max, then a
// prefix sum of per-expert tile counts -- and walks tiles t = blockIdx.x,
// blockIdx.x + gridDim.x, ...  Ragged row tails are handled in the tile
// itself: rows past an expert's end are clamped (forward, dgrad: their
// results are never stored) or read as zero (wgrad, where they would enter
// the sum); stores are predicated per row and column.  So there is no pad
// copy and no output memset (TileOPs issue #1566, "Summary" and "Proposed
// change"), and an expert with no rows costs nothing in forward/dgrad and
// still writes its all-zero dW[g] in wgrad.
//
// MFMA: v_mfma_f32_32x32x16_bf16, fp32 accumulation.  A workgroup is 4 waves
// (2 x 2) over a 256 x 256 output tile; each wave owns 128 x 128, i.e. 4 x 4
// MFMA blocks of 32 x 32 (256 accumulator registers per lane).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gg_internal.h"

namespace gg {

constexpr int BM = 256;          // tile rows
constexpr int BN = 256;          // tile cols
constexpr int BK = 64;           // reduction step
constexpr int NT = 256;          // threads per workgroup (4 waves)
constexpr int STAGE_BYTES = 256 * BK * 2;   // one operand tile: 32 KB

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum Mode { FWD = 0, DGRAD = 1, WGRAD = 2, MASKED = 3 };

struct Params {
  const uint16_t* a;        // forward/masked/wgrad: X;  dgrad: dY
  const uint16_t* b;        // forward/masked/dgrad: W;  wgrad: dY
  const int32_t* groups;    // end offsets, or masked_m
  void* c;                  // output
  int64_t m;                // rows of X (ragged) or max_m (masked)
  int64_t k;
  int64_t n;
  int32_t num_groups;
};

// One operand tile: element (row r, reduction index q) of the tile lives at
// byte origin + 2 (r * ld + q) (red-contig) or origin + 2 (q * ld + r)
// (red-strided).  Loads go through a buffer resource rebuilt per reduction
// step whose record count ends exactly at the last byte the tile may read,
// so rows past an expert's end (and reduction rows past its length) read as
// zero from the hardware range check, and nothing past the operand is ever
// touched.  All offsets are in the 32-bit VGPR offset (the scalar offset is
// kept 0: the range check covers the VGPR and instruction offsets).
struct Operand {
  const uint8_t* origin;
  uint32_t ld_bytes;  // 2 * ld
  int32_t rows;       // red-contig: valid tile rows (>= 1)
  int32_t red;        // valid reduction length
  uint32_t row_tail;  // red-strided: bytes from the tile's first row to the end of a memory row
};

constexpr uint32_t kRsrcWord3 = 0x00020000u;   // gfx9 raw buffer, 32-bit dwords
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset every record count here is below

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, (int)kRsrcWord3);
}

// Values every lane of the wave holds alike (decoded from LDS) moved to
// scalar registers, so buffer resources built from them stay scalar.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// ---- global -> registers ---------------------------------------------------

// Red-contig: thread owns chunk c = tid & 7 (reduction values 8c..8c+7) of
// tile rows tid/8 + 32 j, j = 0..7.  Rows past the valid ones fall outside
// the record range (zero); a chunk past the reduction end is sent out of
// range explicitly (it would otherwise read the next row).
__device__ __forceinline__ void load_contig(const Operand& op, int q0, int tid, u32x4 (&r)[8]) {
  const int c = tid & 7;
  // Past the reduction end the record count is 0 (every load reads zero and
  // touches no memory).
  const uint32_t nrec = q0 < op.red ? (uint32_t)op.rows * op.ld_bytes - 2u * (uint32_t)q0 : 0u;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(op.origin + 2 * (int64_t)q0, nrec);
  uint32_t voff = (uint32_t)(tid >> 3) * op.ld_bytes + 16u * (uint32_t)c;
  if (q0 + 8 * c >= op.red) voff = kOutOfRange;
  const uint32_t step = 32u * op.ld_bytes;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    r[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff + j * step, 0, 0));
}

// Red-strided: thread owns the 8 (reduction) x 8 (row) block with reduction
// block rb = tid & 7 and row block cb = tid >> 3.  Reduction rows past the
// valid length fall outside the record range (zero).  Tile rows past the
// memory row end read neighbouring data or zero; they only feed output rows
// or columns that are never stored.
__device__ __forceinline__ void load_strided(const Operand& op, int q0, int tid, u32x4 (&r)[8]) {
  const int rb = tid & 7;
  const int cb = tid >> 3;
  const int left = op.red - q0;
  const uint32_t nrec = left > 0 ? (uint32_t)(left - 1) * op.ld_bytes + op.row_tail : 0u;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(op.origin + (int64_t)q0 * op.ld_bytes, nrec);
  const uint32_t voff = (uint32_t)(8 * rb) * op.ld_bytes + 16u * (uint32_t)cb;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    r[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff + j * op.ld_bytes, 0, 0));
}

// ---- registers -> LDS --------------------------------------------------------

// LDS tile layout: row r at r * 128 bytes, its 16-byte chunk c at chunk
// position c ^ ((r / 2) mod 8).  The LDS serves 16 lanes (256 bytes) of a
// 16-byte access per cycle; 16 consecutive rows at one logical chunk then
// land on 16 distinct 16-byte bank groups (row parity picks the 128-byte
// half, (r / 2) mod 8 the chunk), so fragment reads are conflict-free, and
// so are row-pair writes of 8 chunks each.
__device__ __forceinline__ uint32_t lds_off(int row, int chunk) {
  return (uint32_t)(row * (BK * 2) + ((chunk ^ ((row >> 1) & 7)) << 4));
}

__device__ __forceinline__ void store_contig(uint8_t* lds, int tid, const u32x4 (&r)[8]) {
  const int c = tid & 7;
  const int row0 = tid >> 3;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = row0 + 32 * j;
    *reinterpret_cast<u32x4*>(lds + lds_off(row, c)) = r[j];
  }
}

// Transpose the 8 x 8 block (r[j] holds reduction index j for 8 consecutive
// rows) so that each of the 8 rows gets its 8 reduction values in one chunk.
// Lanes with an odd row block visit the rows in the order 1, 0, 3, 2, ...:
// each write instruction then covers a row pair of opposite parity across
// 16 lanes, which the LDS serves without bank conflicts.
__device__ __forceinline__ void store_strided(uint8_t* lds, int tid, const u32x4 (&r)[8]) {
  const int rb = tid & 7;
  const int flip = (tid >> 3) & 1;
  const int row0 = 8 * (tid >> 3);
  // byte selectors: low halves (even row) or high halves (odd row)
  const uint32_t sel_even = flip ? 0x07060302u : 0x05040100u;
  const uint32_t sel_odd = flip ? 0x05040100u : 0x07060302u;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int w = s >> 1;                                   // dword holding rows 2w, 2w + 1
    const uint32_t sel = (s & 1) ? sel_odd : sel_even;
    const int qr = s ^ flip;
    u32x4 o;
    o[0] = perm_b32(r[1][w], r[0][w], sel);
    o[1] = perm_b32(r[3][w], r[2][w], sel);
    o[2] = perm_b32(r[5][w], r[4][w], sel);
    o[3] = perm_b32(r[7][w], r[6][w], sel);
    *reinterpret_cast<u32x4*>(lds + lds_off(row0 + qr, rb)) = o;
  }
}

template <bool STRIDED>
__device__ __forceinline__ void load_op(const Operand& op, int q0, int tid, u32x4 (&r)[8]) {
  if constexpr (STRIDED) load_strided(op, q0, tid, r); else load_contig(op, q0, tid, r);
}

template <bool STRIDED>
__device__ __forceinline__ void store_op(uint8_t* lds, int tid, const u32x4 (&r)[8]) {
  if constexpr (STRIDED) store_strided(lds, tid, r); else store_contig(lds, tid, r);
}

// ---- per-chunk forms of the above (for the interleaved main loop) --------------

// Buffer resource and lane offset of one operand for one stage; chunk j is
// at voff + j * step.
struct LoadCtx {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t voff;
  uint32_t step;
};

template <bool STRIDED>
__device__ __forceinline__ LoadCtx load_ctx(const Operand& op, int q0, int tid) {
  LoadCtx c;
  if constexpr (STRIDED) {
    const int rb = tid & 7;
    const int cb = tid >> 3;
    const int left = op.red - q0;
    const uint32_t nrec = left > 0 ? (uint32_t)(left - 1) * op.ld_bytes + op.row_tail : 0u;
    c.rs = make_rsrc(op.origin + (int64_t)q0 * op.ld_bytes, nrec);
    c.voff = (uint32_t)(8 * rb) * op.ld_bytes + 16u * (uint32_t)cb;
    c.step = op.ld_bytes;
  } else {
    const int ch = tid & 7;
    const uint32_t nrec = q0 < op.red ? (uint32_t)op.rows * op.ld_bytes - 2u * (uint32_t)q0 : 0u;
    c.rs = make_rsrc(op.origin + 2 * (int64_t)q0, nrec);
    c.voff = (uint32_t)(tid >> 3) * op.ld_bytes + 16u * (uint32_t)ch;
    if (q0 + 8 * ch >= op.red) c.voff = kOutOfRange;
    c.step = 32u * op.ld_bytes;
  }
  return c;
}

__device__ __forceinline__ u32x4 load_chunk(const LoadCtx& c, int j) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(c.rs, c.voff + j * c.step, 0, 0));
}

// Write chunk j of the staged registers (red-contig: row tid/8 + 32 j;
// red-strided: the j-th of the thread's 8 rows, transposed).
template <bool STRIDED>
__device__ __forceinline__ void store_chunk(uint8_t* lds, int tid, const u32x4 (&r)[8], int j) {
  if constexpr (STRIDED) {
    const int rb = tid & 7;
    const int flip = (tid >> 3) & 1;
    const int row0 = 8 * (tid >> 3);
    const uint32_t sel_even = flip ? 0x07060302u : 0x05040100u;
    const uint32_t sel_odd = flip ? 0x05040100u : 0x07060302u;
    const int w = j >> 1;
    const uint32_t sel = (j & 1) ? sel_odd : sel_even;
    u32x4 o;
    o[0] = perm_b32(r[1][w], r[0][w], sel);
    o[1] = perm_b32(r[3][w], r[2][w], sel);
    o[2] = perm_b32(r[5][w], r[4][w], sel);
    o[3] = perm_b32(r[7][w], r[6][w], sel);
    *reinterpret_cast<u32x4*>(lds + lds_off(row0 + (j ^ flip), rb)) = o;
  } else {
    const int row = (tid >> 3) + 32 * j;
    *reinterpret_cast<u32x4*>(lds + lds_off(row, tid & 7)) = r[j];
  }
}

// ---- MFMA over one staged reduction step ---------------------------------------

__device__ __forceinline__ bf16x8 lds_frag(const uint8_t* lds, int row, int chunk) {
  u32x4 v = *reinterpret_cast<const u32x4*>(lds + lds_off(row, chunk));
  return __builtin_bit_cast(bf16x8, v);
}

// The 4 A and 4 B fragments of one 16-deep MFMA sub-step (ks = 0..3 of a
// 64-deep stage): lane l reads tile row 32 i + l % 32 (plus the wave's
// offset), reduction chunk 2 ks + l / 32.
struct Frags {
  bf16x8 a[4];
  bf16x8 b[4];
};

__device__ __forceinline__ void read_frags(const uint8_t* As, const uint8_t* Bs, int wm, int wn,
                                           int lane, int ks, Frags& f) {
  const int lrow = lane & 31;
  const int chunk = 2 * ks + (lane >> 5);
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = lds_frag(As, 128 * wm + 32 * i + lrow, chunk);
#pragma unroll
  for (int j = 0; j < 4; ++j) f.b[j] = lds_frag(Bs, 128 * wn + 32 * j + lrow, chunk);
}

// Fragment q of a sub-step: q < 4 is A fragment q, else B fragment q - 4.
__device__ __forceinline__ void read_frag(const uint8_t* As, const uint8_t* Bs, int wm, int wn,
                                          int lane, int ks, int q, Frags& f) {
  const int lrow = lane & 31;
  const int chunk = 2 * ks + (lane >> 5);
  if (q < 4) f.a[q] = lds_frag(As, 128 * wm + 32 * q + lrow, chunk);
  else f.b[q - 4] = lds_frag(Bs, 128 * wn + 32 * (q - 4) + lrow, chunk);
}

// LDS-only barrier: this wave's LDS operations are complete, then all waves
// meet.  (Outstanding global loads stay in flight.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16 MFMAs of one sub-step.  The B fragment is the MFMA's first operand, so
// each 32 x 32 result block is C^T and a lane ends up holding 4 consecutive
// output columns of one output row (see store_tile).
__device__ __forceinline__ void mfma_block(const Frags& f, floatx16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

// ---- epilogue --------------------------------------------------------------------

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (round to nearest even) packed in one dword, low
// half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  floatx2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// Accumulator block (i, j) holds C^T: element v of lane l is output row
// 128 wm + 32 i + l % 32 and output column 128 wn + 32 j + 8 (v / 4) +
// 4 (l / 32) + v % 4.  So each lane stores 4 consecutive columns at a time
// (8 bytes of bf16 or 16 bytes of fp32).  Stores go through a buffer
// resource ending at the tile's last valid element: rows past the valid ones
// are dropped by the range check; a group of 8 columns past the valid ones
// (cols is a multiple of 8) is skipped for the whole wave.
template <bool OUT_F32>
__device__ __forceinline__ void store_tile(uint8_t* cbase, uint32_t ldc_bytes, int rows, int cols,
                                           int wm, int wn, int lane, const floatx16 (&acc)[4][4]) {
  constexpr uint32_t esz = OUT_F32 ? 4 : 2;
  const uint32_t nrec = (uint32_t)(rows - 1) * ldc_bytes + (uint32_t)cols * esz;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(cbase, nrec);
  const uint32_t lane_off = (uint32_t)(128 * wm + (lane & 31)) * ldc_bytes +
                            (uint32_t)(128 * wn + 4 * (lane >> 5)) * esz;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t voff = lane_off + (uint32_t)(32 * i) * ldc_bytes;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int col8 = 128 * wn + 32 * j + 8 * rr;      // first of 8 columns, wave-uniform
        if (col8 >= cols) continue;
        const uint32_t imm = (uint32_t)(32 * j + 8 * rr) * esz;
        const floatx16& a = acc[i][j];
        if constexpr (OUT_F32) {
          // Built as a float vector and bit-cast whole: a u32x4 built from
          // per-element bit casts of accumulator values was miscompiled by
          // this hipcc (every lane of the vector got element 0).
          floatx4 v = {a[4 * rr + 0], a[4 * rr + 1], a[4 * rr + 2], a[4 * rr + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, voff + imm, 0, 0);
        } else {
          u32x2 v = {pack_bf16x2(a[4 * rr + 0], a[4 * rr + 1]), pack_bf16x2(a[4 * rr + 2], a[4 * rr + 3])};
          __builtin_amdgcn_raw_buffer_store_b64(v, rs, voff + imm, 0, 0);
        }
      }
    }
  }
}

// ---- group decode (prologue) ---------------------------------------------------

// Block-wide inclusive scan of one int per thread (sum or max).
template <bool MAX>
__device__ __forceinline__ int block_scan_incl(int v, int* scratch, int tid) {
  scratch[tid] = v;
  __syncthreads();
#pragma unroll
  for (int d = 1; d < NT; d <<= 1) {
    int o = tid >= d ? scratch[tid - d] : (MAX ? 0 : 0);
    __syncthreads();
    if (tid >= d) v = MAX ? (v > o ? v : o) : v + o;
    scratch[tid] = v;
    __syncthreads();
  }
  return v;
}

// Fills s_start/s_end with the clamped row range of every group and, unless
// WGRAD, s_pref[0..E] with the exclusive prefix of per-group row-tile counts.
template <int MODE>
__device__ void decode_groups(const Params& p, int32_t* s_start, int32_t* s_end, int32_t* s_pref,
                              int* scratch, int tid) {
  const int E = p.num_groups;
  const int per = (E + NT - 1) / NT;
  const int g0 = tid * per;
  const int g1 = g0 + per < E ? g0 + per : E;
  if constexpr (MODE == MASKED) {
    for (int g = g0; g < g1; ++g) {
      int a = p.groups[g];
      a = a < 0 ? 0 : a;
      a = a > p.m ? (int)p.m : a;
      s_start[g] = 0;
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
    const int incl = block_scan_incl<true>(run, scratch, tid);
    int before = 0;
    if (tid > 0) before = scratch[tid - 1];
    (void)incl;
    __syncthreads();
    const int mcap = (int)p.m;
    for (int g = g0; g < g1; ++g) {
      int e = s_end[g] > before ? s_end[g] : before;
      s_end[g] = e < mcap ? e : mcap;
    }
    __syncthreads();
    for (int g = g0; g < g1; ++g) s_start[g] = g == 0 ? 0 : s_end[g - 1];
  }
  __syncthreads();
  if constexpr (MODE != WGRAD) {
    int local = 0;
    for (int g = g0; g < g1; ++g) local += (s_end[g] - s_start[g] + BM - 1) / BM;
    const int incl = block_scan_incl<false>(local, scratch, tid);
    int run = incl - local;
    for (int g = g0; g < g1; ++g) {
      s_pref[g] = run;
      run += (s_end[g] - s_start[g] + BM - 1) / BM;
    }
    if (tid == NT - 1) s_pref[E] = incl;
    __syncthreads();
  }
}

// Largest g in [0, E) with s_pref[g] <= t (s_pref is non-decreasing,
// s_pref[0] = 0 <= t).
__device__ __forceinline__ int find_group(const int32_t* s_pref, int E, int t) {
  int lo = 0, hi = E;          // invariant: s_pref[lo] <= t < s_pref[hi] (s_pref[E] = total)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (s_pref[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// ---- the kernel ------------------------------------------------------------------

template <int MODE, bool OUT_F32>
__global__ __launch_bounds__(NT, 1) void grouped_gemm_kernel(Params p) {
  constexpr bool A_STRIDED = (MODE == WGRAD);
  constexpr bool B_STRIDED = (MODE != DGRAD);

  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * STAGE_BYTES];
  __shared__ int32_t s_start[GG_MAX_GROUPS_DEV];
  __shared__ int32_t s_end[GG_MAX_GROUPS_DEV];
  __shared__ int32_t s_pref[GG_MAX_GROUPS_DEV + 1];
  __shared__ int s_scan[NT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);     // wave index, held in a scalar register
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int E = p.num_groups;

  decode_groups<MODE>(p, s_start, s_end, s_pref, s_scan, tid);

  // Output tile grid.
  const int64_t out_cols = (MODE == DGRAD) ? p.k : p.n;
  const int col_tiles = (int)((out_cols + BN - 1) / BN);
  int64_t total;
  int row_tiles_w = 0;
  if constexpr (MODE == WGRAD) {
    row_tiles_w = (int)((p.k + BM - 1) / BM);
    total = (int64_t)E * row_tiles_w * col_tiles;
  } else {
    total = (int64_t)uniform(s_pref[E]) * col_tiles;
  }

  // LDS: [A stage 0][A stage 1][B stage 0][B stage 1].
  auto As = [&](int st) { return smem + st * STAGE_BYTES; };
  auto Bs = [&](int st) { return smem + (2 + st) * STAGE_BYTES; };

  constexpr uint32_t esz = OUT_F32 ? 4 : 2;
  const uint8_t* pa = reinterpret_cast<const uint8_t*>(p.a);
  const uint8_t* pb = reinterpret_cast<const uint8_t*>(p.b);
  uint8_t* pc = reinterpret_cast<uint8_t*>(p.c);

  for (int64_t t = blockIdx.x; t < total; t += gridDim.x) {
    Operand A, B;
    uint8_t* cbase;
    uint32_t ldc_bytes;
    int out_rows, out_cols_valid;
    {
      const int ct = (int)(t % col_tiles);
      const int64_t rt_all = t / col_tiles;
      const int col0 = ct * BN;
      if constexpr (MODE == WGRAD) {
        const int g = (int)(rt_all / row_tiles_w);
        const int rt = (int)(rt_all % row_tiles_w);
        const int row0 = rt * BM;                 // first k index of the tile
        const int s = uniform(s_start[g]), e = uniform(s_end[g]);
        // A(row kk, red i) = X[s + i, row0 + kk]
        A.origin = pa + 2 * ((int64_t)s * p.k + row0);
        A.ld_bytes = (uint32_t)(2 * p.k);
        A.rows = (int)(p.k - row0 < BM ? p.k - row0 : BM);
        A.red = e - s;
        A.row_tail = (uint32_t)(2 * (p.k - row0));
        // B(row n, red i) = dY[s + i, col0 + n]
        B.origin = pb + 2 * ((int64_t)s * p.n + col0);
        B.ld_bytes = (uint32_t)(2 * p.n);
        B.rows = (int)(p.n - col0 < BN ? p.n - col0 : BN);
        B.red = e - s;
        B.row_tail = (uint32_t)(2 * (p.n - col0));
        ldc_bytes = (uint32_t)(esz * p.n);
        cbase = pc + esz * ((int64_t)g * p.k * p.n + (int64_t)row0 * p.n + col0);
        out_rows = A.rows;
        out_cols_valid = B.rows;
      } else {
        const int g = uniform(find_group(s_pref, E, (int)rt_all));
        const int rt = (int)rt_all - uniform(s_pref[g]);
        const int s = uniform(s_start[g]), e = uniform(s_end[g]);
        const int row0 = s + rt * BM;             // first expert row of the tile
        const int rows = (e - row0) < BM ? (e - row0) : BM;
        const int64_t arow = (MODE == MASKED) ? (int64_t)g * p.m + row0 : (int64_t)row0;
        if constexpr (MODE == DGRAD) {
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
          ldc_bytes = (uint32_t)(esz * p.k);
          cbase = pc + esz * (arow * p.k + col0);
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
          ldc_bytes = (uint32_t)(esz * p.n);
          cbase = pc + esz * (arow * p.n + col0);
        }
        out_rows = rows;
        out_cols_valid = B.rows;
      }
    }

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int red = A.red;
    const int nk = (red + BK - 1) / BK;
    if (nk > 0) {
      // Software pipeline, one LDS barrier per 64-deep stage kt (LDS buffer
      // cur = kt & 1).  On entry to stage kt: LDS[cur] holds stage kt,
      // registers ra/rb hold stage kt+1 (loaded during stage kt-1) and
      // fragment set f[0] holds sub-step 0 of stage kt.  The 64 MFMAs of the
      // stage are issued in order; beside MFMA m the wave issues:
      //   m  0..7  : read sub-step 1 fragment m -> f[1]; write A chunk m of stage kt+1
      //   m  8..15 : write B chunk m-8 of stage kt+1; load A chunk m-8 of stage kt+2
      //   m 16..23 : read sub-step 2 fragment -> f[0]; load B chunk of stage kt+2
      //   m 32..39 : read sub-step 3 fragment -> f[1]
      //   m 47     : LDS barrier (stage kt+1 is written, stage kt no longer read)
      //   m 48..55 : read sub-step 0 of stage kt+1 (LDS[cur^1]) -> f[0]
      // Scheduling barriers keep the compiler from regrouping these.  Loads
      // past the reduction end read zeros without touching memory; what they
      // put in LDS is never read for this tile.
      u32x4 ra[8], rb[8];
      {
        const LoadCtx ca = load_ctx<A_STRIDED>(A, 0, tid);
        const LoadCtx cb = load_ctx<B_STRIDED>(B, 0, tid);
#pragma unroll
        for (int j = 0; j < 8; ++j) ra[j] = load_chunk(ca, j);
#pragma unroll
        for (int j = 0; j < 8; ++j) rb[j] = load_chunk(cb, j);
#pragma unroll
        for (int j = 0; j < 8; ++j) store_chunk<A_STRIDED>(As(0), tid, ra, j);
#pragma unroll
        for (int j = 0; j < 8; ++j) store_chunk<B_STRIDED>(Bs(0), tid, rb, j);
        const LoadCtx ca1 = load_ctx<A_STRIDED>(A, BK, tid);
        const LoadCtx cb1 = load_ctx<B_STRIDED>(B, BK, tid);
#pragma unroll
        for (int j = 0; j < 8; ++j) ra[j] = load_chunk(ca1, j);
#pragma unroll
        for (int j = 0; j < 8; ++j) rb[j] = load_chunk(cb1, j);
      }
      lds_barrier();
      Frags f[2];
      read_frags(As(0), Bs(0), wm, wn, lane, 0, f[0]);
      for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const uint8_t* Ac = As(cur);
        const uint8_t* Bc = Bs(cur);
        uint8_t* An = As(cur ^ 1);
        uint8_t* Bn = Bs(cur ^ 1);
        const LoadCtx ca = load_ctx<A_STRIDED>(A, (kt + 2) * BK, tid);
        const LoadCtx cb = load_ctx<B_STRIDED>(B, (kt + 2) * BK, tid);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 64; ++m) {
          const int ks = m >> 4;
          const int q = m & 15;
          Frags& fc = f[ks & 1];
          const int i = q >> 2, j = q & 3;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fc.b[j], fc.a[i], acc[i][j], 0, 0, 0);
          if (ks == 0) {
            if (q < 8) {
              read_frag(Ac, Bc, wm, wn, lane, 1, q, f[1]);
              store_chunk<A_STRIDED>(An, tid, ra, q);
            } else {
              store_chunk<B_STRIDED>(Bn, tid, rb, q - 8);
              ra[q - 8] = load_chunk(ca, q - 8);
            }
          } else if (ks == 1) {
            if (q < 8) {
              read_frag(Ac, Bc, wm, wn, lane, 2, q, f[0]);
              rb[q] = load_chunk(cb, q);
            }
          } else if (ks == 2) {
            if (q < 8) read_frag(Ac, Bc, wm, wn, lane, 3, q, f[1]);
            if (q == 15) lds_barrier();
          } else {
            if (q < 8) read_frag(An, Bn, wm, wn, lane, 0, q, f[0]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // The last stage's reads are done; the next tile's prologue rewrites LDS.
      lds_barrier();
    }
    store_tile<OUT_F32>(cbase, ldc_bytes, out_rows, out_cols_valid, wm, wn, lane, acc);
  }
}

// ---- host-side launchers -------------------------------------------------------

template <int MODE, bool OUT_F32>
static hipError_t launch_one(const Params& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((grouped_gemm_kernel<MODE, OUT_F32>), dim3(grid), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_mode(const Params& p, bool out_f32, int grid, hipStream_t stream) {
  return out_f32 ? launch_one<MODE, true>(p, grid, stream) : launch_one<MODE, false>(p, grid, stream);
}

// Upper bound on the number of output tiles, from host-known sizes only
// (the device knows the exact count).  Each expert adds at most one partial
// row tile beyond ceil(rows / BM).
static int64_t max_tiles(int mode, int64_t m, int64_t k, int64_t n, int64_t E) {
  if (mode == WGRAD) return E * ((k + BM - 1) / BM) * ((n + BN - 1) / BN);
  const int64_t cols = mode == DGRAD ? k : n;
  const int64_t ct = (cols + BN - 1) / BN;
  if (mode == MASKED) return E * ((m + BM - 1) / BM) * ct;
  return ((m + BM - 1) / BM + E) * ct;
}

hipError_t launch(int mode, const void* a, const void* b, const int32_t* groups, void* c,
                  bool out_f32, int64_t m, int64_t k, int64_t n, int32_t num_groups,
                  int num_cus, hipStream_t stream) {
  Params p;
  p.a = static_cast<const uint16_t*>(a);
  p.b = static_cast<const uint16_t*>(b);
  p.groups = groups;
  p.c = c;
  p.m = m;
  p.k = k;
  p.n = n;
  p.num_groups = num_groups;
  const int64_t tiles = max_tiles(mode, m, k, n, num_groups);
  if (tiles <= 0) return hipSuccess;
  const int grid = (int)(tiles < num_cus ? tiles : num_cus);
  switch (mode) {
    case FWD: return launch_mode<FWD>(p, out_f32, grid, stream);
    case DGRAD: return launch_mode<DGRAD>(p, out_f32, grid, stream);
    case WGRAD: return launch_mode<WGRAD>(p, out_f32, grid, stream);
    case MASKED: return launch_mode<MASKED>(p, out_f32, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gg
