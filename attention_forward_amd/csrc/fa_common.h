// Shared device code of the gfx950 attention kernels: operand types, MFMA
// wrappers, LDS swizzles, tile loads and the per-tile S / softmax / PV step.
//
// Orientation.  Scores are computed transposed, S^T = K Q^T, and the output as
// O^T = V^T P^T, with v_mfma_f32_32x32x16_{f16,bf16}.  In the 32x32 accumulator
// lane l holds column n = l % 32 and rows 8*(r/4) + 4*(l/32) + r%4 of register
// r, so every lane owns one query (n) and a slice of keys (S^T) or of head
// dimensions (O^T).  Row max and row sum of the softmax are then in-lane
// reductions plus one exchange between lanes l and l ^ 32, and the per-query
// rescale and 1/l normalisation are per-lane scalars.  The S^T accumulator of
// one 32-key block holds, per lane, the 16 keys that two 16-deep PV steps take
// as their B operand (P^T), in the key order of the accumulator; V^T is read in
// that same key order with the transposing LDS read ds_read_b64_tr_b16, so the
// contraction over keys pairs every p_j with its own v_j.  (On the RTX 5090 the
// score fragment already has the layout the PV operand wants -- "The FA5090
// Optimization Journey", sec. 2.3 -- on CDNA the transposed orientation and the
// transposing read play that role.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

constexpr int KT = 64;  // keys per K/V tile
constexpr int LOG2_KT = 6;
static_assert(KT == 1 << LOG2_KT, "tiles of a power-of-two key count");

// Geometry of one head dimension HD (64 or 128): a K or V row is HD 16-bit
// elements, read in 16-byte slots; a direct-to-LDS load instruction moves a
// 1 KiB chunk of whole rows.
template <int HD>
struct Geom {
  static_assert(HD == 64 || HD == 128, "head dimensions 64 and 128");
  static constexpr int ROW = HD * 2;            // bytes per row
  static constexpr int SLOTS = ROW / 16;        // 16-byte slots per row
  static constexpr int TILE = KT * ROW;         // bytes per K or V tile
  static constexpr int RPC = 1024 / ROW;        // rows per 1 KiB load chunk
  static constexpr int CHUNKS = TILE / 1024;    // load chunks per tile
  static constexpr int DSTEPS = HD / 16;        // 16-deep d-steps of S^T = K Q^T
  static constexpr int DBLOCKS = HD / 32;       // 32-wide d-blocks of O^T
  static constexpr int KOPS = 2 * DSTEPS;       // K operands per tile (2 key blocks)
  static constexpr int VOPS = 4 * DBLOCKS;      // V^T operands per tile (4 key steps)
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((__vector_size__(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

#define ATTN_LDS __attribute__((address_space(3)))
// Build-time switches (defaults are the measured best):
// ATTN_KDEPTH: K operand reads issued ahead of their MFMA.
// ATTN_FAST_SOFTMAX: try the max-free form of the threshold rule first on
//   tiles every row sees in full (softmax_fast).
// ATTN_SETPRIO: raise the prefill MFMA phase's wave priority; with the
//   shorter max-free softmax phase it measured 1-2% slower than leaving the
//   two waves of a SIMD at equal priority.
#ifndef ATTN_KDEPTH
#define ATTN_KDEPTH 8
#endif
#ifndef ATTN_FAST_SOFTMAX
#define ATTN_FAST_SOFTMAX 1
#endif
#ifndef ATTN_SETPRIO
#define ATTN_SETPRIO 0
#endif

// dtype 0: IEEE binary16, dtype 1: bfloat16
template <int DT>
__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == 0)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Round two floats to the 16-bit dtype (round to nearest even) and pack them.
template <int DT>
__device__ __forceinline__ unsigned pack2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  if constexpr (DT == 0)
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2));
  else
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

// Value of x in lane l ^ 32 combined with x: returns (x_lo, x_hi) pair per lane.
__device__ __forceinline__ void swap_halves(float x, float& mine, float& other) {
  int xi = __builtin_bit_cast(int, x);
  auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  // lanes 0-31: r[0] = own value, r[1] = value of lane + 32
  // lanes 32-63: r[0] = value of lane - 32, r[1] = own value
  float a = __builtin_bit_cast(float, (int)r[0]);
  float b = __builtin_bit_cast(float, (int)r[1]);
  const bool lo = (threadIdx.x & 32) == 0;
  mine = lo ? a : b;
  other = lo ? b : a;
}

__device__ __forceinline__ float half_max(float x) {
  int xi = __builtin_bit_cast(int, x);
  auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}

__device__ __forceinline__ float half_sum(float x) {
  int xi = __builtin_bit_cast(int, x);
  auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

// ---- LDS swizzles (16-byte slots) ----
// The 64 banks of 4 bytes span 256 bytes: one row at HD = 128, two rows at
// HD = 64.
// K is read 16 bytes per lane, 32 consecutive rows at one slot.  HD = 128:
// XOR the slot with the low 4 row bits so 16 consecutive rows hit distinct
// banks.  HD = 64: rows of equal parity share a bank half, so XOR with row
// bits 1-3, which differ across the 8 rows of each parity among 16.
template <int HD>
__device__ __forceinline__ int k_swz(int row) {
  if constexpr (HD == 128)
    return row & 15;
  else
    return (row >> 1) & 7;
}
// V is read with the 8-byte transposing read: each 16-lane group covers 4
// consecutive rows x 32 bytes, and two groups the same rows at the next 32
// bytes.  HD = 128: XOR with f(row & 3) = 2a ^ 8(a & 1) spreads those rows
// over distinct 32-byte bank groups (bits 1-2) and distinct 64-byte groups
// (bits 2-3).  HD = 64: rows r and r + 2 share a bank half; XOR with 4 for
// row bit 1 moves one of them to the other 64 bytes of that half.
template <int HD>
__device__ __forceinline__ int v_swz(int row) {
  if constexpr (HD == 128) {
    int a = row & 3;
    return (a << 1) ^ ((a & 1) << 3);
  } else {
    return ((row >> 1) & 1) << 2;
  }
}

// ---- HBM -> LDS tile load ----
// One wave instruction of a direct-to-LDS load moves 64 x 16 B into 1 KiB of
// LDS at base + 16*lane, i.e. RPC full rows.  The lane that fills LDS slot p
// of row r reads global slot p ^ swz(r) of that row, so LDS slot s ^ swz(r)
// holds the row's logical slot s.
// Per-lane byte offset, within a 1 KiB load chunk, of the 16-byte source slot
// the lane fetches: row (chunk*RPC + lane/SLOTS), slot (lane%SLOTS) ^ swz(row).
// A chunk index that advances by a multiple of 16 rows keeps the row bits the
// swizzles use, so one offset serves all of a lane's chunks that far apart.
template <int HD, bool IS_V>
__device__ __forceinline__ unsigned load_lane_offset(int chunk) {
  using G = Geom<HD>;
  const int lane = threadIdx.x & 63;
  const int r = chunk * G::RPC + lane / G::SLOTS;
  const int slot = (lane % G::SLOTS) ^ (IS_V ? v_swz<HD>(r) : k_swz<HD>(r));
  return (unsigned)(r * G::ROW + slot * 16);
}

// ---- bounds-checked buffer loads ----
// A raw buffer descriptor covers [base, base + bytes); a lane whose byte offset
// falls outside reads zeros (into registers, or into LDS for the direct-to-LDS
// form), so ragged tails need neither clamping nor branches.  bytes < 2^32.
constexpr unsigned RSRC_WORD3 = 0x00020000u;  // gfx9 raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long long bytes) {
  const int n = bytes <= 0 ? 0 : (int)(unsigned)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, RSRC_WORD3);
}

// 64 lanes x 16 bytes from rsrc at byte offsets voff -> LDS dst + 16 * lane
// Cache policy of a load (the buffer instructions' cache-policy operand):
// CP_NT marks a streaming, non-temporal read, for data read exactly once.
constexpr int CP_DEFAULT = 0;
constexpr int CP_NT = 2;

template <int CP = CP_DEFAULT>
__device__ __forceinline__ void load_chunk(__amdgpu_buffer_rsrc_t r, unsigned voff,
                                           unsigned char ATTN_LDS* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, reinterpret_cast<ATTN_LDS void*>(dst), 16, (int)voff,
                                           0, 0, CP);
}

__device__ __forceinline__ u32x4 load_b128(__amdgpu_buffer_rsrc_t r, unsigned voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

// 16 bytes per lane to rsrc at byte offset voff; offsets past the range are dropped
__device__ __forceinline__ void store_b128(__amdgpu_buffer_rsrc_t r, unsigned voff, u32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(x, r, (int)voff, 0, 0);
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).  Issued
// through the builtin so the compiler's own wait bookkeeping sees it.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void vm_wait_all() { vm_wait<0>(); }

// ---- LDS operand reads with immediate offsets and data-dependent waits ----
// The reads are issued through inline asm so that the compiler neither hoists
// them nor inserts a wait on the direct-to-LDS loads of the next tile (which
// write the other buffer); each consumer first executes an s_waitcnt that
// takes the loaded registers as operands, so it cannot be scheduled before it.
template <int OFF>
__device__ __forceinline__ u32x4 lds_b128(unsigned addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x2 lds_tr16(unsigned addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4& x) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "n"(N));
}
__device__ __forceinline__ void lds_write_b64(unsigned addr, u32x2 x) {
  asm volatile("ds_write_b64 %0, %1" : : "v"(addr), "v"(x) : "memory");
}
// every LDS access issued so far has completed
__device__ __forceinline__ void lgkm_drain() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Per-lane LDS byte addresses (relative to a K/V stage) that stay fixed for
// the whole key loop; tile, stage and step offsets are immediates.  Entries
// past the head dimension's d-steps and d-blocks are unused.
struct LaneAddr {
  unsigned k[8];  // K operand of d-step st (key block 0; block 1 is +32 rows)
  unsigned v[4];  // V^T operand of d-block db (key step 0; others are row offsets)
};
// The swizzles only permute 16-byte slots within a row, and the slot index of
// d-step st (d-block db) differs from that of d-step 0 (d-block 0) in the bits
// that st (db) XORs in: k[st] = k[0] ^ (st << 5), and v[db] = v[0] ^ (db <<
// VSH) with VSH 6 for the 16-bit layouts (4 slots per d-block) and 5 for FP8
// (2 slots).  Stage bases are multiples of 1 KiB, so the XOR commutes with
// adding the stage base: with ATTN_COMPACT_LA the kernels keep only k[0] and
// v[0] in registers and form the others with one XOR per read, in place of
// the add of the base they need anyway.
#ifndef ATTN_COMPACT_LA
#define ATTN_COMPACT_LA 1
#endif
// k0 / v0: base + k[0] (base + v[0]) formed once per tile step; the empty asm
// makes it opaque, so that the compiler cannot fold the XOR constants into
// the lane address and keep every d-step's address in a register again.
// COMPACT selects the form per caller: the 16-bit steps use it (ATTN_COMPACT_LA),
// the FP8 steps keep every address in a register (the compact form measured
// 1.3% slower there).
template <bool COMPACT = ATTN_COMPACT_LA>
__device__ __forceinline__ unsigned lane_base(unsigned base, unsigned lane_addr) {
  unsigned a = base + lane_addr;
  if (COMPACT) asm volatile("" : "+v"(a));
  return a;
}
template <bool COMPACT = ATTN_COMPACT_LA>
__device__ __forceinline__ unsigned kaddr(unsigned k0, const LaneAddr& la, unsigned base, int st) {
  return COMPACT ? (k0 ^ (unsigned)(st << 5)) : base + la.k[st];
}
template <int VSH, bool COMPACT = ATTN_COMPACT_LA>
__device__ __forceinline__ unsigned vaddr(unsigned v0, const LaneAddr& la, unsigned base, int db) {
  return COMPACT ? (v0 ^ (unsigned)(db << VSH)) : base + la.v[db];
}

template <int HD>
__device__ __forceinline__ LaneAddr lane_addresses() {
  using G = Geom<HD>;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5, n = lane & 31, j = lane & 15, h = (lane >> 4) & 1;
  LaneAddr a = {};
#pragma unroll
  for (int st = 0; st < G::DSTEPS; ++st)
    a.k[st] = (unsigned)(n * G::ROW + (((2 * st + g) ^ k_swz<HD>(n)) * 16));
  // V^T reads: rows 4g + (j>>2) (+16t, +32kb, +8 for items 4..7), 32-byte column
  // group 4db + 2h, 8-byte half (j&3)>>1 ... see v_swz
  const int row_l = 4 * g + (j >> 2);
#pragma unroll
  for (int db = 0; db < G::DBLOCKS; ++db) {
    const int slot = 4 * db + 2 * h + ((j & 3) >> 1);
    a.v[db] = (unsigned)(row_l * G::ROW + ((slot ^ v_swz<HD>(row_l)) * 16) + 8 * (j & 1));
  }
  return a;
}

// ---- FP8 (OCP E4M3) operands at head dimension 128 ----
// A row is 128 bytes, so tiles, loads and the K reads are those of the 16-bit
// layout at head dimension 64 (Geom<64>).  Both matrix products use
// v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales: a lane holds 32
// bytes of each operand, and A and B use the same byte -> k order, so any
// consistent assignment of the 64 k values to (lane half, byte) is exact.
//
// V is read with the byte-transposing read ds_read_b64_tr_b8: in each 16-lane
// group, lane 8u + i receives byte i of the 8 bytes addressed by lanes u, 2+u,
// ..., 14+u, one from each.  So a group's lanes address 8 keys (rows) at two
// 8-byte column offsets, and each destination lane ends up with one column
// (one d) of 8 keys.  XOR of the 16-byte slot with 2 * (row bit 1) + 4 * (row
// bit 3) puts the 8 rows of a 32-lane pass on distinct banks.
__device__ __forceinline__ int v_swz8(int row) {
  return (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2);
}

template <bool IS_V>
__device__ __forceinline__ unsigned load_lane_offset8(int chunk) {
  using G = Geom<64>;
  const int lane = threadIdx.x & 63;
  const int r = chunk * G::RPC + lane / G::SLOTS;
  const int slot = (lane % G::SLOTS) ^ (IS_V ? v_swz8(r) : k_swz<64>(r));
  return (unsigned)(r * G::ROW + slot * 16);
}

// k[st]: K operand half st (16-byte slot 2st + g of row n), as at d = 64 in 16
// bits; the FP8 k-step st8 uses halves 2st8 and 2st8 + 1.  v[db]: the byte
// address this lane supplies to the transposing reads of d-block db: key row
// 8(x>>3) + 4(h>>1) + ((x>>1)&3) (+16 per read), column 32db + 16(h&1) +
// 8(x&1), with h = lane>>4, x = lane&15.  The keys so read for destination
// lane half g are 16t + 8(e>>2) + 4g + (e&3), e = 0..7, in read t: exactly the
// keys whose scores the lane holds in accumulator elements 8t' + e of key
// block t>>1 (t' = t&1), in the order store_p packs them.
__device__ __forceinline__ LaneAddr lane_addresses8() {
  LaneAddr a = lane_addresses<64>();
  const int lane = threadIdx.x & 63;
  const int h = lane >> 4, x = lane & 15;
  const int row = 8 * (x >> 3) + 4 * (h >> 1) + ((x >> 1) & 3);
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int slot = 2 * db + (h & 1);
    a.v[db] = (unsigned)(row * 128 + ((slot ^ v_swz8(row)) * 16) + 8 * (x & 1));
  }
  return a;
}

__device__ __forceinline__ f32x16 mfma8(const u32x8& a, const u32x8& b, f32x16 c) {
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  // format 0 (E4M3) for both operands, block scales 2^(127 - 127) = 1
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a),
                                                         __builtin_bit_cast(i32x8, b), c, 0, 0,
                                                         0, 127, 0, 127);
}

template <int OFF>
__device__ __forceinline__ u32x2 lds_tr8(unsigned addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int N>
__device__ __forceinline__ void lgkm_wait8(u32x8& x) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "n"(N));
}

// S^T = K Q^T in FP8: 2 key blocks x 2 k-steps of 64 d; all eight K reads are
// issued first, each operand waited for just before its MFMA.
template <int QB>
__device__ __forceinline__ void qk_step8(unsigned kbase, const LaneAddr& la,
                                         const u32x8 (&qf)[QB][2], f32x16 (&s)[2][QB]) {
  u32x8 ko[4];
  const unsigned k0 = lane_base<false>(kbase, la.k[0]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kb = i >> 1, st = i & 1;
    u32x4 lo, hi;
    if (kb == 0) {
      lo = lds_b128<0>(kaddr<false>(k0, la, kbase, 2 * st));
      hi = lds_b128<0>(kaddr<false>(k0, la, kbase, 2 * st + 1));
    } else {
      lo = lds_b128<32 * 128>(kaddr<false>(k0, la, kbase, 2 * st));
      hi = lds_b128<32 * 128>(kaddr<false>(k0, la, kbase, 2 * st + 1));
    }
    ko[i] = u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    switch (i) {
      case 0: lgkm_wait8<6>(ko[0]); break;
      case 1: lgkm_wait8<4>(ko[1]); break;
      case 2: lgkm_wait8<2>(ko[2]); break;
      default: lgkm_wait8<0>(ko[3]); break;
    }
    const int kb = i >> 1, st = i & 1;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      s[kb][qb] = mfma8(ko[i], qf[qb][st], st == 0 ? f32x16{} : s[kb][qb]);
  }
}

// O^T += V^T P^T in FP8: 4 d-blocks, one MFMA of all 64 keys each; an operand
// is four transposing reads (keys 16t .. 16t+15 of the lane half), two
// operands in flight.
template <int QB>
__device__ __forceinline__ void pv_step8(unsigned vbase, const LaneAddr& la,
                                         const u32x8 (&pf)[QB], f32x16 (&o)[4][QB]) {
  u32x8 vo[2];
  const unsigned v0 = lane_base<false>(vbase, la.v[0]);
  auto read_v = [&](int db, u32x8& dst) {
    const unsigned a = vaddr<5, false>(v0, la, vbase, db);
    const u32x2 r0 = lds_tr8<0>(a), r1 = lds_tr8<16 * 128>(a), r2 = lds_tr8<32 * 128>(a),
                r3 = lds_tr8<48 * 128>(a);
    dst = u32x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
  };
  read_v(0, vo[0]);
  read_v(1, vo[1]);
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    u32x8& cur = vo[db & 1];
    if (db < 3)
      lgkm_wait8<4>(cur);
    else
      lgkm_wait8<0>(cur);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) o[db][qb] = mfma8(cur, pf[qb], o[db][qb]);
    if (db + 2 < 4) read_v(db + 2, vo[db & 1]);
  }
}

// ---- the three parts of one 64-key tile, for QB blocks of 32 queries ----
//
// qf: Q^T operands [QB][DSTEPS] (16-deep d steps).  s: S^T accumulators [2 key
// blocks][QB].  o: O^T accumulators [DBLOCKS d-blocks][QB].  m: reference max
// (log2 units, -inf initially); l: this lane's running sum over its half of
// the keys.  key0: global index of the tile's first key; qrow0: global index
// of the wave's first query.  Online softmax across tiles: "The FA5090
// Optimization Journey", sec. 2.6 (exp2 with log2 e folded into the scale,
// running max in the log2 domain) and sec. 2.8 (effective max of a fully
// masked tile); "10 rounds of hand-written fused attention ...", round R8 (m
// and l carried).

// S^T = K Q^T: 2 key blocks x DSTEPS d-steps; K operands read KD steps ahead.
// kbase: LDS address of the K tile.
template <int DT, int QB, int HD>
__device__ __forceinline__ void qk_step(unsigned kbase, const LaneAddr& la,
                                        const u32x4 (&qf)[QB][Geom<HD>::DSTEPS],
                                        f32x16 (&s)[2][QB]) {
  using G = Geom<HD>;
  constexpr int DS = G::DSTEPS, N = G::KOPS;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
  constexpr int KD = ATTN_KDEPTH < N ? ATTN_KDEPTH : N;
  u32x4 ko[KD];
  const unsigned k0 = lane_base(kbase, la.k[0]);
  auto read_k = [&](int i, u32x4& dst) {
    // i = kb * DS + st (cases past N are never taken)
#define ATTN_KREAD(I)                                                                  \
  case I:                                                                              \
    dst = lds_b128<((I) / DS) * 32 * G::ROW>(kaddr(k0, la, kbase, (I) % DS));         \
    break;
    switch (i) {
      ATTN_KREAD(0) ATTN_KREAD(1) ATTN_KREAD(2) ATTN_KREAD(3) ATTN_KREAD(4) ATTN_KREAD(5)
      ATTN_KREAD(6) ATTN_KREAD(7) ATTN_KREAD(8) ATTN_KREAD(9) ATTN_KREAD(10) ATTN_KREAD(11)
      ATTN_KREAD(12) ATTN_KREAD(13) ATTN_KREAD(14) ATTN_KREAD(15)
    }
#undef ATTN_KREAD
  };
#pragma unroll
  for (int i = 0; i < KD; ++i) read_k(i, ko[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    u32x4& cur = ko[i % KD];
    // reads issued so far: min(N, KD + i); read i is done when at most
    // (issued - i - 1) younger ones are outstanding
    switch (i + KD < N ? KD - 1 : N - 1 - i) {
      case 7: lgkm_wait<7>(cur); break;
      case 6: lgkm_wait<6>(cur); break;
      case 5: lgkm_wait<5>(cur); break;
      case 4: lgkm_wait<4>(cur); break;
      case 3: lgkm_wait<3>(cur); break;
      case 2: lgkm_wait<2>(cur); break;
      case 1: lgkm_wait<1>(cur); break;
      default: lgkm_wait<0>(cur); break;
    }
    const int kb = i / DS, st = i % DS;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma<DT>(cur, qf[qb][st], s[kb][qb]);
    if (i + KD < N) read_k(i + KD, ko[i % KD]);
  }
}

// The P^T operand of one tile, written eight weights at a time: w[0..7] are
// the weights of accumulator elements 8t .. 8t+7 of key block kb.
// 16-bit MFMA: pf[kb][t][qb] holds them rounded to the dtype, two per register.
template <int DT, int QB>
__device__ __forceinline__ void store_p(u32x4 (&pf)[2][2][QB], int kb, int t, int qb,
                                        const float (&w)[8]) {
  u32x4 x;
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = pack2<DT>(w[2 * e], w[2 * e + 1]);
  pf[kb][t][qb] = x;
}
// FP8 MFMA: pf[qb] holds all 32 weights of the tile as E4M3 bytes, byte
// 16kb + 8t + e for element 8t + e of key block kb (round to nearest even;
// the weights are at most 1 against the exact running max, inside the range).
template <int DT, int QB>
__device__ __forceinline__ void store_p(u32x8 (&pf)[QB], int kb, int t, int qb,
                                        const float (&w)[8]) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(w[0], w[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(w[2], w[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(w[4], w[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(w[6], w[7], hi, true);
  pf[qb][4 * kb + 2 * t] = (unsigned)lo;
  pf[qb][4 * kb + 2 * t + 1] = (unsigned)hi;
}

// Online softmax of one S^T tile: scores -> P^T operands pf (rounded to the
// dtype), rescaled O and updated m, l.  MASK: apply the key-validity and
// causal test per score (tiles that cross the diagonal or the end of the keys
// only; "The FA5090 Optimization Journey", sec. 2.8, mask specialisation).
//
// Lazy reference max: a lane keeps m unless this tile's max exceeds it by more
// than TAU (log2 units), so p = exp2(x - m) <= 2^TAU; any finite reference
// gives the same O = sum p v / sum p and LSE = m + log2 l (the cancelling 1/l
// of sec. 2.6; the threshold skip of sec. 3).  When m stays, alpha is exactly
// 1 and the multiply leaves O unchanged.  The multiply itself is unconditional:
// a branch around it makes the register allocator move the whole accumulator
// between two homes on every iteration, which costs more than it saves.
//
// With E4M3 weights (FP8 P fragments) the reference is the exact running max
// (tau = 0): the E4M3 rounding of P is relative, so a weight of a row's top
// key taken against a lagging reference lies between grid points and carries
// up to 1/16 relative error, where against the exact max it is exactly 1.  On
// a row dominated by a few keys that error reaches O almost undiminished
// (measured on a CPU model of the kernel: about twice the mean row error of
// rounding against the exact max).  In 16-bit the same offset costs at most
// 2^-9 of a weight, so the lazy rule stays there.
//
// RESCALE_O = false leaves O alone and instead reports, as the return value,
// whether any lane of the wave moved a finite reference max (the only case in
// which O must be multiplied by alpha: a row whose max was -inf has O = 0).
// The caller then applies alpha itself; until that happens alpha is exactly 1
// for every lane, so skipping the multiply changes no bit.

// threshold of the lazy reference max (log2 units) for a P fragment type
template <typename PF>
struct RescaleTau {
  static constexpr float value = 8.0f;
};
template <int N>
struct RescaleTau<u32x8[N]> {
  static constexpr float value = 0.0f;  // E4M3 weights: the exact running max
};

template <int DT, int QB, bool MASK, bool RESCALE_O = true, int NDB = 4, typename PF>
__device__ __forceinline__ bool softmax_step(f32x16 (&s)[2][QB], f32x16 (&o)[NDB][QB],
                                             float (&m)[QB], float (&l)[QB],
                                             PF& pf, float scale_log2, int key0,
                                             int qrow0, int n_keys, bool causal, int causal_off,
                                             float (&alpha_out)[QB]) {
  bool moved = false;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  const int n = lane & 31;
  // Score r of key block kb holds key key0 + 4g + off(kb, r), with the
  // compile-time offset off = 32kb + 8(r >> 2) + (r & 3).  The key is hidden iff
  // key >= n_keys or (causal) key > qi + causal_off, i.e. iff off > lim[qb]
  // with lim = min(n_keys - 1, causal ? qi + causal_off : n_keys - 1) - key0 - 4g:
  // one compare per score against a per-lane limit taken once per tile.
  int lim[QB];
  if constexpr (MASK) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qi = qrow0 + 32 * qb + n;
      const int last = causal ? min(n_keys - 1, qi + causal_off) : n_keys - 1;
      lim[qb] = last - key0 - 4 * g;
    }
  }
  auto hidden = [&](int kb, int qb, int r) {
    return 32 * kb + 8 * (r >> 2) + (r & 3) > lim[qb];
  };
  if constexpr (MASK) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (hidden(kb, qb, r)) s[kb][qb][r] = -INFINITY;
  }
  constexpr float TAU = RescaleTau<PF>::value;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float mx = fmaxf(s[0][qb][0], s[0][qb][1]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = (kb == 0 ? 2 : 0); r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
    mx = half_max(mx);
    // -inf * 0 would be NaN when scale is 0; a fully hidden tile keeps m
    float mxs = mx * scale_log2;
    if constexpr (MASK) mxs = (mx == -INFINITY) ? -INFINITY : mxs;
    const bool jump = mxs > m[qb] + TAU;
    // exp2(0) = 1 exactly when m stays, exp2(-inf) = 0 when m leaves -inf; no
    // branch, so the whole step stays one basic block for the scheduler
    const float alpha = __builtin_amdgcn_exp2f(jump ? m[qb] - mxs : 0.0f);
    moved |= jump && m[qb] != -INFINITY;
    m[qb] = jump ? mxs : m[qb];
    l[qb] *= alpha;
    alpha_out[qb] = alpha;
    if constexpr (RESCALE_O) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db][qb] *= alpha;
    }
    // effective max of a row that has seen no visible key yet ("The FA5090
    // Optimization Journey", sec. 2.8): exp2(-inf - 0) = 0 keeps it NaN-free
    const float m_eff = (m[qb] == -INFINITY) ? 0.0f : m[qb];
    // the row sum adds the fp32 values before they are rounded for the MFMA, so
    // the LSE is that of the exact weights
    float rs = l[qb];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][r], scale_log2, -m_eff));
        if constexpr (MASK) p = hidden(kb, qb, r) ? 0.0f : p;  // exact zero even for scale 0
        s[kb][qb][r] = p;
        rs += p;
      }
    l[qb] = rs;
    // P rounded to the MFMA's input format (RNE)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = s[kb][qb][8 * t + e];
        store_p<DT, QB>(pf, kb, t, qb, w);
      }
  }
  if constexpr (RESCALE_O)
    return false;
  else
    return __builtin_amdgcn_ballot_w64(moved) != 0;
}

// Fast form of the threshold rule for a tile that every row sees in full:
// the weights are taken against the current reference max m, without the
// row max.  Returns true, for the whole wave, when the tile must go through
// softmax_step instead: some row's m is still -inf, or some weight may have
// reached 2^(TAU - 1).  Otherwise no row's max exceeds m + TAU - 1, so
// softmax_step would have kept m with alpha = 1, and l and pf now hold
// exactly what it would have produced (same products, same exponentials,
// same order of the row sum).
//
// The test needs no max: the row sum only grows as it adds non-negative
// weights, so a weight p >= 2^(TAU - 1) leaves rs >= fl(l + p) >=
// fl(l + 2^(TAU - 1)); rs below that bound thus rules out every such weight.
// An infinite or NaN sum fails the test as well.  ("The FA5090 Optimization
// Journey", sec. 3, threshold rescale; the bound on the weights is what keeps
// the fp32 sums and the rounded P in range.)
template <int DT, int QB, typename PF>
__device__ __forceinline__ bool softmax_fast(const f32x16 (&s)[2][QB], const float (&m)[QB],
                                             float (&l)[QB], PF& pf, float scale_log2) {
  constexpr float BOUND = 128.0f;  // 2^(TAU - 1) with TAU = 8
  bool bad = false;
  float rs_q[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float neg_m = -m[qb];
    float rs = l[qb];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          w[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][8 * t + e], scale_log2, neg_m));
          rs += w[e];
        }
        store_p<DT, QB>(pf, kb, t, qb, w);
      }
    bad |= !(rs < l[qb] + BOUND);
    rs_q[qb] = rs;
  }
  const bool redo = __builtin_amdgcn_ballot_w64(bad) != 0;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) l[qb] = redo ? l[qb] : rs_q[qb];
  return redo;
}

// O^T += V^T P^T: DBLOCKS d-blocks x 4 key steps, operands 4 steps ahead.
// Step i: db = i >> 2, kb = (i >> 1) & 1, t = i & 1; the operand's two
// transposing reads cover keys 32kb + 16t + 4g + {0..3} and the same + 8.
// vbase: LDS address of the V tile.
template <int DT, int QB, int HD>
__device__ __forceinline__ void pv_step(unsigned vbase, const LaneAddr& la,
                                        const u32x4 (&pf)[2][2][QB],
                                        f32x16 (&o)[Geom<HD>::DBLOCKS][QB]) {
  using G = Geom<HD>;
  constexpr int N = G::VOPS;
  u32x4 vo[4];
  const unsigned v0 = lane_base(vbase, la.v[0]);
  auto read_v = [&](int i, u32x4& dst) {
    u32x2 lo, hi;
    // cases past N are never taken
#define ATTN_VREAD(I)                                                                  \
  case I:                                                                              \
    lo = lds_tr16<(32 * (((I) >> 1) & 1) + 16 * ((I) & 1)) * G::ROW>(                  \
        vaddr<6>(v0, la, vbase, (I) >> 2));                                            \
    hi = lds_tr16<(32 * (((I) >> 1) & 1) + 16 * ((I) & 1) + 8) * G::ROW>(              \
        vaddr<6>(v0, la, vbase, (I) >> 2));                                            \
    break;
    switch (i) {
      ATTN_VREAD(0) ATTN_VREAD(1) ATTN_VREAD(2) ATTN_VREAD(3) ATTN_VREAD(4) ATTN_VREAD(5)
      ATTN_VREAD(6) ATTN_VREAD(7) ATTN_VREAD(8) ATTN_VREAD(9) ATTN_VREAD(10) ATTN_VREAD(11)
      ATTN_VREAD(12) ATTN_VREAD(13) ATTN_VREAD(14) ATTN_VREAD(15)
    }
#undef ATTN_VREAD
    dst = u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
#pragma unroll
  for (int i = 0; i < 4; ++i) read_v(i, vo[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    u32x4& cur = vo[i & 3];
    // two reads per operand; operands issued so far: min(N, 4 + i)
    switch (i + 4 < N ? 6 : 2 * (N - 1 - i)) {
      case 6: lgkm_wait<6>(cur); break;
      case 4: lgkm_wait<4>(cur); break;
      case 2: lgkm_wait<2>(cur); break;
      default: lgkm_wait<0>(cur); break;
    }
    const int db = i >> 2, kb = (i >> 1) & 1, t = i & 1;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) o[db][qb] = mfma<DT>(cur, pf[kb][t][qb], o[db][qb]);
    if (i + 4 < N) read_v(i + 4, vo[i & 3]);
  }
}

}  // namespace attn
