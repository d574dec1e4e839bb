// Prefill / full forward kernel: one workgroup per (batch*head, block of FWD_BR
// query rows); FWD_NW waves, each owning FWD_QB blocks of 32 query rows whose
// Q^T operands stay in registers for the whole key loop.  K and V tiles of 64
// keys stream HBM -> LDS with direct-to-LDS loads, double buffered so tile j+1
// is in flight while tile j is consumed ("G5: Pipeline 重构与双缓冲", V21: the
// load of the next tile overlaps the compute of the current one; "Three kernels
// for a chip the ecosystem skipped", Kernel one: double-buffered K/V).
//
// Causal: only tiles up to the last key visible to the workgroup's last row are
// loaded; a wave skips the tiles that are fully hidden for all of its rows, and
// only tiles that cross the diagonal (or the end of the keys) pay for the
// per-score test ("The FA5090 Optimization Journey", sec. 2.7 causal skip and
// sec. 2.8 mask specialisation).  Work items are issued heaviest first (largest
// query block index first), the LPT order of sec. 2.7.
#include "fa_common.h"
#include "launch.h"

namespace attn {

template <int DT, int QB, int NW>
__global__ __launch_bounds__(NW * 64, FWD_WAVES_PER_SIMD) void fa_fwd_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            uint16_t* __restrict__ o,
                                                            float* __restrict__ lse, int Hq,
                                                            int Hkv, int Sq, int Sk, int causal,
                                                            float scale_log2, int n_bh, int n_qt) {
  constexpr int BR = NW * QB * 32;
  constexpr int CHUNKS_PER_WAVE = (KT / 4) / NW;  // 1 KiB load instructions per tile per wave
  static_assert((KT / 4) % NW == 0, "tile rows must split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * 2 * TILE_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;
  const int n = lane & 31;

  const int t = blockIdx.x;
  const int rank = t / n_bh;
  const int bh = t - rank * n_bh;
  const int qt = causal ? (n_qt - 1 - rank) : rank;
  const int b = bh / Hq;
  const int hq = bh - b * Hq;
  const int hkv = hq / (Hq / Hkv);

  const uint16_t* qh = q + (size_t)bh * Sq * D;
  const uint16_t* kh = k + ((size_t)b * Hkv + hkv) * Sk * D;
  const uint16_t* vh = v + ((size_t)b * Hkv + hkv) * Sk * D;
  const int causal_off = Sk - Sq;

  const int q0 = qt * BR;
  const int qw0 = q0 + wave * QB * 32;  // this wave's first query row

  // keys this workgroup needs
  int kv_end = Sk;
  if (causal) {
    const int last_q = min(q0 + BR, Sq) - 1;
    kv_end = min(Sk, max(0, last_q + causal_off + 1));
  }
  const int n_tiles = (kv_end + KT - 1) / KT;

  // Q^T operands: lane holds Q[row][16*st + 8*g .. +7] for its query n; rows
  // past Sq read as zeros
  u32x4 qf[QB][8];
  {
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qh, (long long)Sq * ROW);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const unsigned row_off = (unsigned)((qw0 + 32 * qb + n) * ROW + 16 * g);
#pragma unroll
      for (int st = 0; st < 8; ++st) qf[qb][st] = load_b128(qr, row_off + 32 * st);
    }
  }
  f32x16 acc[4][QB];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db][qb] = f32x16{};
  }

  // lane offsets of this wave's load chunks: chunk c*NW + wave covers rows
  // 16c + 4*wave + lane/16, so the swizzle pattern is the same for every c
  static_assert(NW == 4, "one lane offset per wave needs chunks 16 rows apart");
  const unsigned koff = load_lane_offset<false>(wave);
  const unsigned voff = load_lane_offset<true>(wave);
  auto issue_tile = [&](int j) {
    unsigned char ATTN_LDS* base = (unsigned char ATTN_LDS*)(smem) + (j & 1) * 2 * TILE_BYTES;
    const int key0 = j * KT;
    const long long bytes = (long long)(Sk - key0) * ROW;  // keys past Sk read as zeros
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kh + (size_t)key0 * D, bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vh + (size_t)key0 * D, bytes);
#pragma unroll
    for (int c = 0; c < CHUNKS_PER_WAVE; ++c)
      load_chunk(kr, koff + c * 16 * ROW, base + (c * NW + wave) * 1024);
#pragma unroll
    for (int c = 0; c < CHUNKS_PER_WAVE; ++c)
      load_chunk(vr, voff + c * 16 * ROW, base + TILE_BYTES + (c * NW + wave) * 1024);
  };

  const int wave_last_q = min(qw0 + QB * 32, Sq) - 1;
  const bool wave_active = qw0 < Sq;
  const LaneAddr la = lane_addresses();
  const unsigned smem_base = (unsigned)(size_t)(unsigned char ATTN_LDS*)(smem);

  if (n_tiles > 0) issue_tile(0);
  for (int j = 0; j < n_tiles; ++j) {
    vm_wait_all();
    __syncthreads();
    if (j + 1 < n_tiles) issue_tile(j + 1);
    const int key0 = j * KT;
    const bool hidden = causal && key0 > wave_last_q + causal_off;
    if (wave_active && !hidden) {
      const bool need_mask =
          (key0 + KT > Sk) || (causal && key0 + KT - 1 > qw0 + causal_off);
      const unsigned base = smem_base + (unsigned)((j & 1) * 2 * TILE_BYTES);
      if (need_mask)
        tile_step<DT, QB, true>(base, la, qf, acc, m, l, scale_log2, key0, qw0, Sk, causal != 0,
                                causal_off);
      else
        tile_step<DT, QB, false>(base, la, qf, acc, m, l, scale_log2, key0, qw0, Sk, false, 0);
    }
  }

  // epilogue: O = acc / l, rounded to the dtype; LSE = ln2 * (m + log2 l)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = half_sum(l[qb]);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    const int row = qw0 + 32 * qb + n;
    if (row < Sq) {
      uint16_t* orow = o + ((size_t)bh * Sq + row) * D;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int d0 = 32 * db + 8 * jj + 4 * g;
          u32x2 w;
          w[0] = pack2<DT>(acc[db][qb][4 * jj + 0] * inv, acc[db][qb][4 * jj + 1] * inv);
          w[1] = pack2<DT>(acc[db][qb][4 * jj + 2] * inv, acc[db][qb][4 * jj + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + d0) = w;
        }
      if (lse != nullptr && g == 0)
        lse[(size_t)bh * Sq + row] =
            lt > 0.0f ? 0.69314718055994531f * (m[qb] + __builtin_amdgcn_logf(lt)) : -INFINITY;
    }
  }
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  const int n_bh = a.B * a.Hq;
  const int n_qt = (a.Sq + FWD_BR - 1) / FWD_BR;
  const long long items = (long long)n_bh * n_qt;
  dim3 grid((unsigned)items), block(FWD_NW * 64);
  auto q = static_cast<const uint16_t*>(a.q);
  auto k = static_cast<const uint16_t*>(a.k);
  auto v = static_cast<const uint16_t*>(a.v);
  auto o = static_cast<uint16_t*>(a.o);
  if (a.dtype == 0)
    hipLaunchKernelGGL((fa_fwd_kernel<0, FWD_QB, FWD_NW>), grid, block, 0, stream, q, k, v, o,
                       a.lse, a.Hq, a.Hkv, a.Sq, a.Sk, a.causal, a.scale_log2, n_bh, n_qt);
  else
    hipLaunchKernelGGL((fa_fwd_kernel<1, FWD_QB, FWD_NW>), grid, block, 0, stream, q, k, v, o,
                       a.lse, a.Hq, a.Hkv, a.Sq, a.Sk, a.causal, a.scale_log2, n_bh, n_qt);
  return hipGetLastError();
}

}  // namespace attn
