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

constexpr int D = 128;          // head dimension handled by these kernels (HEAD_DIM)
constexpr int KT = 64;          // keys per K/V tile
constexpr int ROW = D * 2;      // bytes per K/V row in LDS (16-bit elements)
constexpr int TILE_BYTES = KT * ROW;  // 16 KiB per K or V tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((__vector_size__(8)));

#define ATTN_LDS __attribute__((address_space(3)))

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
  if constexpr (DT == 0) {
    _Float16 a = (_Float16)lo, b = (_Float16)hi;
    return (unsigned)__builtin_bit_cast(unsigned short, a) |
           ((unsigned)__builtin_bit_cast(unsigned short, b) << 16);
  } else {
    __bf16 a = (__bf16)lo, b = (__bf16)hi;
    return (unsigned)__builtin_bit_cast(unsigned short, a) |
           ((unsigned)__builtin_bit_cast(unsigned short, b) << 16);
  }
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

// ---- LDS swizzles (16-byte slots, 16 slots per 256-byte row) ----
// K is read 16 bytes per lane, 32 consecutive rows at one slot: XOR the slot
// with the low 4 row bits so 8 or 16 consecutive rows hit distinct banks.
__device__ __forceinline__ int k_swz(int row) { return row & 15; }
// V is read with the 8-byte transposing read: each 16-lane group covers 4
// consecutive rows x 32 bytes.  XOR with f(row & 3) = 2a ^ 8(a & 1) spreads those
// rows over distinct 32-byte bank groups (bits 1-2) and distinct 64-byte groups
// (bits 2-3).
__device__ __forceinline__ int v_swz(int row) {
  int a = row & 3;
  return (a << 1) ^ ((a & 1) << 3);
}

// ---- HBM -> LDS tile load ----
// One wave instruction of global_load_lds moves 64 x 16 B into 1 KiB of LDS at
// base + 16*lane, i.e. 4 full rows.  The lane that fills LDS slot p of row r
// reads global slot p ^ swz(r) of that row, so LDS slot s ^ swz(r) holds the
// row's logical slot s.  Rows past the last valid key are clamped to it (their
// scores are masked, their values stay finite).
template <bool IS_V>
__device__ __forceinline__ void load_rows_1k(const uint16_t* src_head, int key_base, int chunk,
                                             int last_key, unsigned char ATTN_LDS* tile) {
  const int lane = threadIdx.x & 63;
  const int r = chunk * 4 + (lane >> 4);
  const int p = lane & 15;
  int key = key_base + r;
  key = key > last_key ? last_key : key;
  const int slot = p ^ (IS_V ? v_swz(r) : k_swz(r));
  const unsigned char* g =
      reinterpret_cast<const unsigned char*>(src_head) + (size_t)key * ROW + slot * 16;
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(g),
                                   reinterpret_cast<ATTN_LDS void*>(tile + chunk * 1024), 16, 0,
                                   0);
}

__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---- one 64-key tile for QB blocks of 32 queries owned by this wave ----
//
// kt, vt: LDS tiles (swizzled).  qf: Q^T operands [QB][8] (16-deep d steps).
// o: O^T accumulators [4 d-blocks][QB].  m: running max (log2 units, -inf
// initially); l: this lane's partial running sum (the lane's half of the keys).
// key0: global index of the tile's first key; qrow0: global index of this
// wave's first query; mask: apply the key-validity / causal test per score.
// Online softmax across tiles: "The FA5090 Optimization Journey", sec. 2.6
// (exp2 with log2 e folded into the scale, running max in the log2 domain,
// sec. 2.8 for the effective max of a fully masked tile); "10 rounds of
// hand-written fused attention ...", round R8 (m and l carried across tiles).
template <int DT, int QB>
__device__ __forceinline__ void tile_step(const unsigned char ATTN_LDS* kt,
                                          const unsigned char ATTN_LDS* vt, const u32x4 (&qf)[QB][8],
                                          f32x16 (&o)[4][QB], float (&m)[QB], float (&l)[QB],
                                          float scale_log2, bool mask, int key0, int qrow0,
                                          int n_keys, bool causal, int causal_off) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  const int n = lane & 31;

  // S^T = K Q^T : two 32-key blocks x QB query blocks, 8 steps of 16 d.
  f32x16 s[2][QB];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
    const int row = 32 * kb + n;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int slot = (2 * st + g) ^ k_swz(row);
      u32x4 a = *reinterpret_cast<const ATTN_LDS u32x4*>(kt + row * ROW + slot * 16);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma<DT>(a, qf[qb][st], s[kb][qb]);
    }
  }

  // visibility of the score in register r of key block kb for query block qb
  auto hidden = [&](int kb, int qb, int r) {
    const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
    const int qi = qrow0 + 32 * qb + n;
    return key >= n_keys || (causal && key > qi + causal_off);
  };
  if (mask) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (hidden(kb, qb, r)) s[kb][qb][r] = -INFINITY;
  }

  // online softmax, per query block
  u32x4 pf[2][2][QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float mx = s[0][qb][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
    mx = half_max(mx);
    // -inf * 0 would be NaN when scale is 0; a fully hidden tile keeps m
    const float mxs = (mx == -INFINITY) ? -INFINITY : mx * scale_log2;
    const float m_new = fmaxf(m[qb], mxs);
    const float m_eff = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m[qb] - m_eff);
    m[qb] = m_new;
    float rs = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][r], scale_log2, -m_eff));
        if (mask && hidden(kb, qb, r)) p = 0.0f;  // exact zero even when scale is 0
        s[kb][qb][r] = p;
        rs += p;
      }
    l[qb] = l[qb] * alpha + rs;
    // alpha == 1 (the max did not move) leaves O bit-identical: skip the
    // multiply when that holds for the whole wave ("The FA5090 Optimization
    // Journey", sec. 2.8, identity rescale-skip decided by a wave-wide vote).
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][qb][r] *= alpha;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack2<DT>(s[kb][qb][8 * t + 2 * e], s[kb][qb][8 * t + 2 * e + 1]);
        pf[kb][t][qb] = w;
      }
  }

  // O^T += V^T P^T : 4 blocks of 32 d x 4 steps of 16 keys.  Operands for step
  // i+1 are read while the MFMA of step i runs.
  const int j = lane & 15;
  const int h = (lane >> 4) & 1;
  // rows 32kb + 16t + 4g + (j>>2) (+8 for the second half); their swizzle only
  // depends on j>>2, so only the d-block changes the slot XOR
  const int row_l = 4 * g + (j >> 2);
  const int sw = v_swz(row_l);
  const unsigned lane_base = (unsigned)(row_l * ROW + 8 * (j & 1));
  auto v_operand_addr = [&](int db) {
    const int slot = 4 * db + 2 * h + ((j & 3) >> 1);
    return lane_base + (unsigned)((slot ^ sw) * 16);
  };
  const unsigned vbase = (unsigned)(size_t)vt;
  u32x4 va[2];
  auto read_v = [&](int step, u32x4& dst) {
    const int db = step >> 2, kb = (step >> 1) & 1, t = step & 1;
    const unsigned addr = vbase + v_operand_addr(db) + (unsigned)((32 * kb + 16 * t) * ROW);
    u32x2 lo, hi;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(lo) : "v"(addr));
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:2048" : "=v"(hi) : "v"(addr));
    dst = u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  read_v(0, va[0]);
#pragma unroll
  for (int step = 0; step < 16; ++step) {
    u32x4& cur = va[step & 1];
    if (step + 1 < 16) {
      read_v(step + 1, va[(step + 1) & 1]);
      asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(cur));
    } else {
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(cur));
    }
    const int db = step >> 2, kb = (step >> 1) & 1, t = step & 1;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) o[db][qb] = mfma<DT>(cur, pf[kb][t][qb], o[db][qb]);
  }
}

}  // namespace attn
