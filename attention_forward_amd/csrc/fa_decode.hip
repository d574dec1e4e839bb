// Single-token decode with split-KV, and the LSE merge of the split partials.
//
// Split kernel: one single-wave workgroup per (batch, kv head, split).  The 32
// query slots of the MFMA tile hold the query heads of the kv head's group (up
// to 32), so each K/V row is read from HBM once for the whole group; the rest
// of the slots are zero and never stored.  The split's keys stream through a
// 32 KiB LDS stage (K and V of 64 keys) whose K and V halves refill as soon as
// they have been read, which keeps bytes in flight for the HBM-bound loop at
// all times (a
// matrix-vector product has an arithmetic intensity near 1 FLOP/B, "The FA5090
// Optimization Journey", sec. 2.3).  The partial output is normalised by its
// own sum and stored in fp32 with its natural-log LSE.
//
// Combine kernel: per (batch, query head), the partials are merged by their
// LSEs, which is the online-softmax rescale of the running state applied across
// splits instead of across tiles ("The FA5090 Optimization Journey", sec. 2.6).
#include "fa_common.h"
#include "launch.h"

namespace attn {

// Residency: each workgroup is launched with DECODE_LDS_BYTES of dynamic LDS,
// twice what its stage needs, so that two workgroups (two streams of K/V
// rows) share a CU.  Measured on the 64 x 8 x 16-split workload: two per CU
// read faster than four (+1.5%) or five (+2%, the count the stage alone
// allows) and than two with the spare LDS used as a second stage.  The LDS is
// requested at launch rather than declared because a static 64 KiB array
// makes the compiler assume one wave per SIMD and move the accumulator into
// AGPRs.
template <int DT, int HD>
__global__ __launch_bounds__(64, 2) void fa_decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ o_part, float* __restrict__ lse_part,
    int Hq, int Hkv, int Sk, int num_splits, float scale_log2) {
  using Gm = Geom<HD>;
  constexpr int D = HD, ROW = Gm::ROW, TILE_BYTES = Gm::TILE;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];  // >= 2 tiles
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  const int n = lane & 31;

  const int t = blockIdx.x;
  const int split = t % num_splits;
  const int bk = t / num_splits;  // b * Hkv + hkv
  const int b = bk / Hkv;
  const int hkv = bk - b * Hkv;
  const int G = Hq / Hkv;

  const int chunk = (Sk + num_splits - 1) / num_splits;
  const int j0 = split * chunk;
  const int j1 = min(Sk, j0 + chunk);

  const uint16_t* kh = k + (size_t)bk * Sk * D;
  const uint16_t* vh = v + (size_t)bk * Sk * D;

  // the group's query heads fill slots 0..G-1; slots past G read as zeros
  u32x4 qf[1][Gm::DSTEPS];
  const bool slot_used = n < G;
  const size_t qrow = (size_t)b * Hq + (size_t)hkv * G + n;  // Sq == 1
  {
    const __amdgpu_buffer_rsrc_t qr =
        make_rsrc(q + ((size_t)b * Hq + (size_t)hkv * G) * D, (long long)G * ROW);
    const unsigned row_off = (unsigned)(n * ROW + 16 * g);
#pragma unroll
    for (int st = 0; st < Gm::DSTEPS; ++st) qf[0][st] = load_b128(qr, row_off + 32 * st);
  }

  f32x16 acc[Gm::DBLOCKS][1];
  float m[1] = {-INFINITY}, l[1] = {0.0f};
#pragma unroll
  for (int db = 0; db < Gm::DBLOCKS; ++db) acc[db][0] = f32x16{};

  unsigned char ATTN_LDS* kt = (unsigned char ATTN_LDS*)(smem);
  unsigned char ATTN_LDS* vt = kt + TILE_BYTES;
  const LaneAddr la = lane_addresses<HD>();
  const unsigned base = (unsigned)(size_t)kt;
  // chunk c covers rows RPC*c + lane/SLOTS: the K swizzle repeats every 16
  // rows (KP chunks), the V swizzle is the same for every chunk
  constexpr int KP = 16 / Gm::RPC;
  unsigned koff[KP];
#pragma unroll
  for (int c = 0; c < KP; ++c) koff[c] = load_lane_offset<HD, false>(c);
  const unsigned voff = load_lane_offset<HD, true>(0);
  // K and V stages refill independently: K(t+1) is issued as soon as QK(t)
  // has read the K stage and V(t+1) as soon as PV(t) has read the V stage, so
  // the next tile's bytes are in flight while this tile is computed.  Loads
  // complete in issue order (K(t), V(t), K(t+1), V(t+1), ...), so "K(t) has
  // landed" is vmcnt <= one tile half (V(t)) and "V(t) has landed" is
  // vmcnt <= one tile half (K(t+1)) or 0 on the last tile.
  // Every K/V byte is read once per call, so the tile loads are marked
  // non-temporal: measured on the 64 x 8 x 16-split workload, 6.1 against
  // 5.7 TB/s with the default cache policy.
  constexpr int HALF = Gm::CHUNKS;  // load instructions per K or V tile
  auto issue_k = [&](int key0) {
    // keys past the split read as zeros
    const __amdgpu_buffer_rsrc_t r = make_rsrc(kh + (size_t)key0 * D, (long long)(j1 - key0) * ROW);
#pragma unroll
    for (int c = 0; c < HALF; ++c)
      load_chunk<CP_NT>(r, koff[c % KP] + (c / KP) * 16 * ROW, kt + c * 1024);
  };
  auto issue_v = [&](int key0) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(vh + (size_t)key0 * D, (long long)(j1 - key0) * ROW);
#pragma unroll
    for (int c = 0; c < HALF; ++c) load_chunk<CP_NT>(r, voff + c * 1024, vt + c * 1024);
  };
  // every LDS read issued so far has returned (the stage may be overwritten)
  auto lds_drained = [] { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };
  if (j0 < j1) {
    issue_k(j0);
    issue_v(j0);
    // Q has landed; K(0) and V(0) may still be in flight.  Tying Q's registers
    // to the wait keeps it after the tile loads and tells the compiler that Q is
    // ready, so it does not wait for every load before the loop.
    if constexpr (Gm::DSTEPS == 8)
      asm volatile("s_waitcnt vmcnt(%8)"
                   : "+v"(qf[0][0]), "+v"(qf[0][1]), "+v"(qf[0][2]), "+v"(qf[0][3]),
                     "+v"(qf[0][4]), "+v"(qf[0][5]), "+v"(qf[0][6]), "+v"(qf[0][7])
                   : "n"(2 * HALF)
                   : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%4)"
                   : "+v"(qf[0][0]), "+v"(qf[0][1]), "+v"(qf[0][2]), "+v"(qf[0][3])
                   : "n"(2 * HALF)
                   : "memory");
  }
  for (int key0 = j0; key0 < j1; key0 += KT) {
    const bool more = key0 + KT < j1;
    f32x16 s[2][1];
    u32x4 pf[2][2][1];
    vm_wait<HALF>();  // K(t)
    qk_step<DT, 1, HD>(base, la, qf, s);
    lds_drained();
    if (more) issue_k(key0 + KT);
    float alpha[1];
    if (key0 + KT > j1)
      softmax_step<DT, 1, true>(s, acc, m, l, pf, scale_log2, key0, 0, j1, false, 0, alpha);
    else
      softmax_step<DT, 1, false>(s, acc, m, l, pf, scale_log2, key0, 0, j1, false, 0, alpha);
    if (more)
      vm_wait<HALF>();  // V(t); K(t+1) may be in flight
    else
      vm_wait_all();
    pv_step<DT, 1, HD>(base + TILE_BYTES, la, pf, acc);
    lds_drained();
    if (more) issue_v(key0 + KT);
  }

  const float lt = half_sum(l[0]);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (slot_used) {
    const size_t prow = qrow * num_splits + split;
    float* op = o_part + prow * D;
#pragma unroll
    for (int db = 0; db < Gm::DBLOCKS; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = 32 * db + 8 * jj + 4 * g;
        float4 w = make_float4(acc[db][0][4 * jj] * inv, acc[db][0][4 * jj + 1] * inv,
                               acc[db][0][4 * jj + 2] * inv, acc[db][0][4 * jj + 3] * inv);
        *reinterpret_cast<float4*>(op + d0) = w;
      }
    if (g == 0)
      lse_part[prow] =
          lt > 0.0f ? 0.69314718055994531f * (m[0] + __builtin_amdgcn_logf(lt)) : -INFINITY;
  }
}

// One wave per (batch, query head) row, COMBINE_ROWS rows per workgroup; lane
// c owns columns HD/64 * c onwards (two at HD = 128, one at HD = 64).  Splits
// are merged COMBINE_BLOCK at a time with
// the online-softmax rescale (running max M, running sum L): a block's partial
// LSEs (wave-uniform, scalar loads) and partial outputs are loaded together, so
// a row costs one memory round trip per block rather than a max pass followed
// by a weighted-sum pass.
constexpr int COMBINE_ROWS = 4;
constexpr int COMBINE_BLOCK = 16;

// partial outputs of one split for this lane's columns (HD / 64 of them)
template <int HD>
__device__ __forceinline__ float2 load_cols(const float* p) {
  if constexpr (HD == 128)
    return *reinterpret_cast<const float2*>(p);
  else
    return make_float2(*p, 0.0f);
}

template <int DT, int HD>
__global__ __launch_bounds__(64 * COMBINE_ROWS) void fa_combine_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    uint16_t* __restrict__ o, float* __restrict__ lse, int rows, int num_splits) {
  constexpr int D = HD, CPL = HD / 64;  // columns per lane
  const int lane = threadIdx.x & 63;
  const unsigned r = blockIdx.x * COMBINE_ROWS + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (r >= (unsigned)rows) return;
  const float* ls = lse_part + (size_t)r * num_splits;
  const float* op = o_part + (size_t)r * num_splits * D + CPL * lane;
  float M = -INFINITY, L = 0.0f, a0 = 0.0f, a1 = 0.0f;
  // merge n splits starting at s whose LSEs are lv and outputs x
  auto merge = [&](const float* lv, const float2* x, int n) {
    float mb = -INFINITY;
    for (int i = 0; i < n; ++i) mb = fmaxf(mb, lv[i]);
    const float mn = fmaxf(M, mb);
    // while every split so far is empty (mn = -inf) shift by 0: every weight
    // is then exp(-inf) = 0, with no branch that would hold back the loads
    const float ref = mn == -INFINITY ? 0.0f : mn;
    const float alpha = __expf(M - ref);  // 0 while M = -inf
    L *= alpha;
    a0 *= alpha;
    a1 *= alpha;
    for (int i = 0; i < n; ++i) {
      const float w = __expf(lv[i] - ref);  // exp(-inf) = 0 for an empty split
      L += w;
      a0 += w * x[i].x;
      a1 += w * x[i].y;
    }
    M = mn;
  };
  int s = 0;
  for (; s + COMBINE_BLOCK <= num_splits; s += COMBINE_BLOCK) {
    float lv[COMBINE_BLOCK];
    float2 x[COMBINE_BLOCK];
#pragma unroll
    for (int i = 0; i < COMBINE_BLOCK; ++i)
      x[i] = load_cols<HD>(op + (size_t)(s + i) * D);
#pragma unroll
    for (int i = 0; i < COMBINE_BLOCK; ++i) lv[i] = ls[s + i];
    merge(lv, x, COMBINE_BLOCK);
  }
  for (; s < num_splits; ++s) {
    const float lv = ls[s];
    const float2 x = load_cols<HD>(op + (size_t)s * D);
    merge(&lv, &x, 1);
  }
  if (L > 0.0f) {
    a0 /= L;
    a1 /= L;
  }
  if constexpr (CPL == 2) {
    *reinterpret_cast<unsigned*>(o + (size_t)r * D + 2 * lane) = pack2<DT>(a0, a1);
  } else {
    const unsigned w = pack2<DT>(a0, 0.0f);
    o[(size_t)r * D + lane] = (uint16_t)(w & 0xffffu);
  }
  if (lse != nullptr && lane == 0) lse[r] = (M == -INFINITY) ? -INFINITY : M + __logf(L);
}

// 64 KiB at either head dimension (two tiles, 32 or 16 KiB, are used; see the kernel)
constexpr unsigned DECODE_LDS_BYTES = 4 * Geom<128>::TILE;

template <int DT, int HD>
static void launch_decode_split_t(const DecodeArgs& a, hipStream_t stream) {
  const long long items = (long long)a.B * a.Hkv * a.num_splits;
  hipLaunchKernelGGL((fa_decode_split_kernel<DT, HD>), dim3((unsigned)items), dim3(64),
                     DECODE_LDS_BYTES, stream, static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                     a.o_part, a.lse_part, a.Hq, a.Hkv, a.Sk, a.num_splits, a.scale_log2);
}

hipError_t launch_decode_split(const DecodeArgs& a, hipStream_t stream) {
  if (a.d == 64)
    a.dtype == 0 ? launch_decode_split_t<0, 64>(a, stream) : launch_decode_split_t<1, 64>(a, stream);
  else
    a.dtype == 0 ? launch_decode_split_t<0, 128>(a, stream)
                 : launch_decode_split_t<1, 128>(a, stream);
  return hipGetLastError();
}

template <int DT, int HD>
static void launch_combine_t(const CombineArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)((a.rows + COMBINE_ROWS - 1) / COMBINE_ROWS)), block(64 * COMBINE_ROWS);
  hipLaunchKernelGGL((fa_combine_kernel<DT, HD>), grid, block, 0, stream, a.o_part, a.lse_part,
                     static_cast<uint16_t*>(a.o), a.lse, a.rows, a.num_splits);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.d == 64)
    a.dtype == 0 ? launch_combine_t<0, 64>(a, stream) : launch_combine_t<1, 64>(a, stream);
  else
    a.dtype == 0 ? launch_combine_t<0, 128>(a, stream) : launch_combine_t<1, 128>(a, stream);
  return hipGetLastError();
}

}  // namespace attn
