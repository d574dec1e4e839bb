// Prefill / full forward kernel.
//
// One workgroup of 8 waves per (batch*head, block of FWD_BR = 256 query rows);
// wave w owns rows 32w..32w+31 and keeps their Q^T operands in registers for
// the whole key loop.  64-key K and V tiles stream HBM -> LDS with
// bounds-checked direct-to-LDS loads into a K ring and a V ring (two or three
// stages each, by input format; see the load hooks below), issued two
// half-steps before their first use ("G5: Pipeline 重构与双缓冲", V21 and V26:
// the next tile's load overlaps the current compute, and K and V have separate
// readiness).
//
// Ping-pong: waves w and w+4 share a SIMD.  Group A (waves 0-3) and group B
// (waves 4-7) alternate between an MFMA phase, [O += P(j-1) V(j-1); S(j) = K(j)
// Q^T], and a VALU phase, [online softmax of S(j)], one workgroup barrier per
// half-step, with B one half-step behind A.  So while one wave of a SIMD
// issues matrix instructions the other runs its exponentials, and the matrix
// pipe is not left idle while a single wave works through its softmax (the
// pages' kernels lean on several resident warps for the same overlap: "The
// FA5090 Optimization Journey", sec. 2.3 and 2.7; "G5", V21).
//
// Causal: only tiles up to the last key visible to the workgroup's last row
// are loaded, a wave computes only the tiles visible to its own rows, and only
// tiles that cross the diagonal (or the end of the keys) pay for the per-score
// test ("The FA5090 Optimization Journey", sec. 2.7 causal skip and sec. 2.8
// mask specialisation).  Work items are issued heaviest first (largest query
// block first), the LPT order of sec. 2.7.
#include <atomic>

#include "fa_common.h"
#include "launch.h"

namespace attn {

static_assert(KT == FWD_KT, "the host's split arithmetic uses the kernels' tile");

// Order of the two products in the MFMA phase of step j.  PV_FIRST: O +=
// P(j-1) V(j-1), then S(j) = K(j) Q^T.  QK_FIRST: S(j) first, so that the
// scores the softmax phase needs are done early, and the products still in
// the matrix pipe when the phase ends (the compiler lets the last products of
// a phase issue after its barrier, since they touch no memory) are P V ones,
// which nothing in the next softmax phase waits for.  Measured (paired):
// QK_FIRST +3.3% to +5.6% for FP8, whose softmax phase is the long one; for
// the 16-bit formats, whose MFMA phase is the long one, -0.2% at d = 128 and
// -6% at d = 64, so they keep PV_FIRST.
enum MfmaOrder { PV_FIRST = 0, QK_FIRST = 1 };

// 1: persistent grid (one workgroup per compute unit, items in a snake
// order); 0: one workgroup per item, dispatched by the hardware.
#ifndef ATTN_PERSIST
#define ATTN_PERSIST 1
#endif
// Each wave writes its rows' output as soon as its last P V product is done,
// in the softmax phase that follows: with the causal mask the waves of a
// diagonal block finish their rows up to three steps apart, so most stores
// complete while the others still compute, and the next item's Q and first K
// tile then wait on fewer stores.  Measured (paired, against writing the
// output after the item's last step): +1.8% causal bf16, +0.9% at S = 32768,
// +7.5% FP8, and +0.4% to +0.9% on non-causal shapes once the output goes out
// through the LDS slice below (-0.5% before, when issuing the stores after
// the next item's loads gained 0.7% there).


// 1: Q in and the 16-bit O out through a per-wave LDS slice (whole rows per
// memory instruction); 0: straight between HBM and the registers.
#ifndef ATTN_STAGE_IO
#define ATTN_STAGE_IO 1
#endif

#ifndef ATTN_XCD_ORDER
#define ATTN_XCD_ORDER 1
#endif

#ifndef ATTN_ORDER16
#define ATTN_ORDER16 0
#endif
#ifndef ATTN_ORDER8
#define ATTN_ORDER8 1
#endif

// Input formats.  In16<DT, HD>: fp16 (DT 0) or bf16 (DT 1) Q, K, V at head
// dimension HD, O in the same dtype.  In8<DT>: OCP E4M3 Q, K, V at head
// dimension 128 with per-tensor descales (Q's and K's folded into the score
// scale on the host, V's applied to O), O in dtype DT.  Each gives the LDS
// layout (Geom of the row size in bytes), the operand fragments and the two
// matrix steps of a tile; the schedule around them is the same.
template <int DT_, int HD_>
struct In16 {
  static constexpr int DT = DT_, HD = HD_, LAYOUT_HD = HD_, DBLOCKS = HD_ / 32;
  static constexpr bool FP8 = false;
  // tile-load scheme (ATTN_LOADERS values, measured per format): both groups
  // in their softmax phases at d = 128 (+2.4%), group B alone at d = 64 (the
  // other scheme loses 9% there)
  static constexpr int LOAD_MODE = HD_ == 128 ? 3 : 1;
  using QFrag = u32x4[1][Geom<HD_>::DSTEPS];
  using PFrag = u32x4[2][2][1];
  // order of the MFMA phase (see MfmaOrder)
  static constexpr int ORDER = ATTN_ORDER16;
  // Q in and O out through the per-wave LDS slice
  static constexpr bool STAGE_IO = ATTN_STAGE_IO;
  // one buffer descriptor per head for the tile loads (see issue below)
  static constexpr bool HEAD_RSRC = true;
  // the softmax phase of the main loops at raised wave priority (see below)
  static constexpr bool PRIO_SOFTMAX = true;
  __device__ static LaneAddr lanes() { return lane_addresses<HD_>(); }
  template <bool IS_V>
  __device__ static unsigned load_offset(int chunk) {
    return load_lane_offset<HD_, IS_V>(chunk);
  }
  // lane holds Q[row][16*st + 8*g .. +7] for its query; row_off: the row's first byte
  __device__ static void load_q(QFrag& qf, __amdgpu_buffer_rsrc_t qr, unsigned row_off) {
    const int g = (threadIdx.x >> 5) & 1;
#pragma unroll
    for (int st = 0; st < Geom<HD_>::DSTEPS; ++st)
      qf[0][st] = load_b128(qr, row_off + 16 * g + 32 * st);
  }
  // the same operands from an LDS copy of the wave's rows laid out as a K tile
  __device__ static void read_q(QFrag& qf, unsigned base, const LaneAddr& la) {
    const unsigned k0 = lane_base(base, la.k[0]);
#pragma unroll
    for (int st = 0; st < Geom<HD_>::DSTEPS; ++st) qf[0][st] = lds_b128<0>(kaddr(k0, la, base, st));
#pragma unroll
    for (int st = 0; st < Geom<HD_>::DSTEPS; ++st) lgkm_wait<0>(qf[0][st]);
  }
  __device__ static void qk(unsigned kbase, const LaneAddr& la, const QFrag& qf,
                            f32x16 (&s)[2][1]) {
    qk_step<DT_, 1, HD_>(kbase, la, qf, s);
  }
  __device__ static void pv(unsigned vbase, const LaneAddr& la, const PFrag& pf,
                            f32x16 (&o)[DBLOCKS][1]) {
    pv_step<DT_, 1, HD_>(vbase, la, pf, o);
  }
};

template <int DT_>
struct In8 {
  static constexpr int DT = DT_, HD = 128, LAYOUT_HD = 64, DBLOCKS = 4;
  static constexpr bool FP8 = true;
  // group A at the start of its MFMA phase, which at twice the 16-bit rate
  // leaves it waiting at the barrier anyway (+2.2% over group B in its softmax
  // phase; both groups in their softmax phases: -1.6%)
  static constexpr int LOAD_MODE = 0;
  using QFrag = u32x8[1][2];
  using PFrag = u32x8[1];
  static constexpr int ORDER = ATTN_ORDER8;
  // the slice measured 2% slower for FP8: Q and O go straight to and from HBM
  static constexpr bool STAGE_IO = false;
  // a descriptor per tile: the per-head form adds vector address arithmetic to
  // the MFMA phase, where group A issues the FP8 loads (measured -4.5%)
  static constexpr bool HEAD_RSRC = false;
  // equal wave priorities (the raised softmax priority measured -0.5% to -1.4%)
  static constexpr bool PRIO_SOFTMAX = false;
  __device__ static LaneAddr lanes() { return lane_addresses8(); }
  template <bool IS_V>
  __device__ static unsigned load_offset(int chunk) {
    return load_lane_offset8<IS_V>(chunk);
  }
  // lane holds Q[row] bytes of slots 4st + g and 4st + 2 + g for k-step st,
  // the halves qk_step8 reads of K
  __device__ static void load_q(QFrag& qf, __amdgpu_buffer_rsrc_t qr, unsigned row_off) {
    const int g = (threadIdx.x >> 5) & 1;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const u32x4 lo = load_b128(qr, row_off + 16 * (4 * st + g));
      const u32x4 hi = load_b128(qr, row_off + 16 * (4 * st + 2 + g));
      qf[0][st] = u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
  __device__ static void read_q(QFrag& qf, unsigned base, const LaneAddr& la) {
    u32x4 h[4];
    const unsigned k0 = lane_base<false>(base, la.k[0]);
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = lds_b128<0>(kaddr<false>(k0, la, base, i));
#pragma unroll
    for (int i = 0; i < 4; ++i) lgkm_wait<0>(h[i]);
#pragma unroll
    for (int st = 0; st < 2; ++st)
      qf[0][st] = u32x8{h[2 * st][0], h[2 * st][1], h[2 * st][2], h[2 * st][3],
                        h[2 * st + 1][0], h[2 * st + 1][1], h[2 * st + 1][2], h[2 * st + 1][3]};
  }
  __device__ static void qk(unsigned kbase, const LaneAddr& la, const QFrag& qf,
                            f32x16 (&s)[2][1]) {
    qk_step8<1>(kbase, la, qf, s);
  }
  __device__ static void pv(unsigned vbase, const LaneAddr& la, const PFrag& pf,
                            f32x16 (&o)[DBLOCKS][1]) {
    pv_step8<1>(vbase, la, pf, o);
  }
};

// PART: split-KV form for grids too small to fill the chip.  Work item
// (q block, batch*head, split s) attends to keys [s * split_keys, (s + 1) *
// split_keys) only and writes the normalised partial O in fp32 and its LSE
// (natural log) to o_part [B*Hq*Sq, n_split, d] and lse_part [B*Hq*Sq,
// n_split]; the split-KV combine merges them.  The kernel body is the same:
// it sees K and V from the split's first key on, Sk cut to the split and the
// causal offset shifted by the split's start.  A split with no visible key
// writes O = 0 and LSE = -inf, which the combine weighs by 0.
// o_scale multiplies O before it is rounded (V's descale in FP8, else 1).
template <typename F, bool PART>
__global__ __launch_bounds__(FWD_NW * 64, 2) void fa_fwd_kernel(
    const unsigned char* __restrict__ q, const unsigned char* __restrict__ k,
    const unsigned char* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse, int Hq,
    int Hkv, int Sq, int Sk_all, int causal, float scale_log2, float o_scale, int n_bh, int n_qt,
    float* __restrict__ o_part, float* __restrict__ lse_part, int n_split, int split_keys,
    int n_items) {
  constexpr int DT = F::DT, HD = F::HD;
  constexpr int NW = FWD_NW;
  constexpr int QB = 1;
  constexpr int BR = FWD_BR;
  static_assert(NW == 8 && FWD_QB == 1, "two groups of four single-block waves");
  // LDS: K stages at [0, 2 tiles), V stages at [2 tiles, 4 tiles); G is the
  // layout of rows of ROW bytes (the 16-bit layout of the same row size)
  using G = Geom<F::LAYOUT_HD>;
  constexpr int D = HD, ROW = G::ROW, TILE_BYTES = G::TILE;
  // which waves issue the tile loads (see below), and ST stages per ring:
  // three for the scheme that loads in both softmax phases, else two
  constexpr int LM = ATTN_LOADERS >= 0 ? ATTN_LOADERS : F::LOAD_MODE;
  constexpr int ST = LM == 3 ? 3 : 2;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * ST * TILE_BYTES];
  // Per-wave staging of the Q block in and of the 16-bit O block out: the
  // wave's 32 rows, laid out as a K tile (16-byte slots XOR-swizzled by row),
  // so that both move between HBM and the wave in whole rows, 1 KiB per
  // instruction, instead of 16- and 8-byte pieces of 32 rows each.
  constexpr int OROW = HD * 2;  // bytes per row of a 16-bit O
  constexpr int SROW = ROW > OROW ? ROW : OROW;
  __shared__ __attribute__((aligned(1024))) unsigned char sio[F::STAGE_IO ? NW * 32 * SROW : 16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool group_a = wave < NW / 2;
  const int g = lane >> 5;
  const int n = lane & 31;
  unsigned char ATTN_LDS* const slice_ptr =
      (unsigned char ATTN_LDS*)(sio) + (F::STAGE_IO ? wave * 32 * SROW : 0);
  const unsigned slice = (unsigned)(size_t)slice_ptr;

  // Persistent: the grid has at most one workgroup per compute unit, and
  // workgroup w takes items w, 2G - 1 - w, 2G + w, 4G - 1 - w, ... (G
  // workgroups), a snake over the heaviest-first item order, so that with
  // causal items (cost falling with the item index) every workgroup's total
  // stays close to the mean.  Between items the workgroup keeps running:
  // no dispatch gap, and the next item's loads start as soon as the last
  // one's LDS reads are done (every wave has passed the final barrier).
  f32x16 acc[F::DBLOCKS][QB];
  float m[QB], l[QB];
  // epilogue of an item: O = acc / l, rounded to the dtype; LSE = ln2 * (m + log2 l)
  auto epilogue = [&](int bh, int qw0, int sp) {
    // the slice's address, opaque here so that the compiler forms the lane
    // addresses when they are needed instead of keeping them in registers
    // (or spilling them) across the key loop
    unsigned sl = slice;
    asm volatile("" : "+s"(sl));
    if constexpr (PART) {
      const float lt = half_sum(l[0]);
      const float inv = lt > 0.0f ? o_scale / lt : 0.0f;
      const int row = qw0 + n;
      if (row < Sq) {
        const size_t prow = ((size_t)bh * Sq + row) * n_split + sp;
        float* orow = o_part + prow * D;
#pragma unroll
        for (int db = 0; db < F::DBLOCKS; ++db)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int d0 = 32 * db + 8 * jj + 4 * g;
            f32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = acc[db][0][4 * jj + e] * inv;
            *reinterpret_cast<f32x4*>(orow + d0) = w;
          }
        if (g == 0)
          lse_part[prow] =
              lt > 0.0f ? 0.69314718055994531f * (m[0] + __builtin_amdgcn_logf(lt)) : -INFINITY;
      }
    } else {
      const float lt = half_sum(l[0]);
      const float inv = lt > 0.0f ? o_scale / lt : 0.0f;
      const int row = qw0 + n;
      if constexpr (F::STAGE_IO) {
        // lane (n, g) holds row n, 16-byte slot 4db + jj, half g: into the
        // slice (slot x of row r at x ^ swz(r)), then back out as whole rows,
        // RPI rows per instruction; rows past Sq fall outside the store's
        // range and are dropped.  The slot bits lie below the row bits, so
        // each address is a per-lane base XOR a constant (bases opaque, as
        // for sl, so that the compiler keeps two registers, not 24).
        unsigned wb = sl + n * OROW + (k_swz<HD>(n) << 4) + 8 * g;
        asm volatile("" : "+v"(wb));
#pragma unroll
        for (int db = 0; db < F::DBLOCKS; ++db)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            u32x2 w;
            w[0] = pack2<DT>(acc[db][0][4 * jj + 0] * inv, acc[db][0][4 * jj + 1] * inv);
            w[1] = pack2<DT>(acc[db][0][4 * jj + 2] * inv, acc[db][0][4 * jj + 3] * inv);
            lds_write_b64(wb ^ ((4 * db + jj) << 4), w);
          }
        // read side: lane L covers row r = RPI i + r0 (r0 = L / LPR), slot
        // x = L % LPR, i.e. LDS slot x ^ swz(r); swz(r) = swz(r0) ^ c(i),
        // c(i) = 4 (i & 3) at d = 128 (swz = row & 15) and 4 (i & 1) at d = 64
        // (swz = (row >> 1) & 7), and the row step is 1 KiB, an immediate
        constexpr int LPR = OROW / 16, RPI = 64 / LPR, NI = 32 / RPI;
        const int r0 = lane / LPR, x = lane % LPR;
        unsigned rb = sl + r0 * OROW + ((x ^ k_swz<HD>(r0)) << 4);
        asm volatile("" : "+v"(rb));
        u32x4 ob[NI];
#define ATTN_OREAD(I)                                                                 \
  if ((I) < NI)                                                                      \
    ob[(I) < NI ? (I) : 0] =                                                         \
        lds_b128<(I) * 1024>(rb ^ ((HD == 128 ? ((I) & 3) : ((I) & 1)) << 6));
        ATTN_OREAD(0) ATTN_OREAD(1) ATTN_OREAD(2) ATTN_OREAD(3) ATTN_OREAD(4) ATTN_OREAD(5)
        ATTN_OREAD(6) ATTN_OREAD(7)
#undef ATTN_OREAD
        const __amdgpu_buffer_rsrc_t orr =
            make_rsrc(o + ((size_t)bh * Sq + qw0) * D, (long long)(Sq - qw0) * OROW);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          lgkm_wait<0>(ob[i]);
          store_b128(orr, (unsigned)((RPI * i + r0) * OROW + x * 16), ob[i]);
        }
      } else if (row < Sq) {
        uint16_t* orow = o + ((size_t)bh * Sq + row) * D;
#pragma unroll
        for (int db = 0; db < F::DBLOCKS; ++db)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int d0 = 32 * db + 8 * jj + 4 * g;
            u32x2 w;
            w[0] = pack2<DT>(acc[db][0][4 * jj + 0] * inv, acc[db][0][4 * jj + 1] * inv);
            w[1] = pack2<DT>(acc[db][0][4 * jj + 2] * inv, acc[db][0][4 * jj + 3] * inv);
            *reinterpret_cast<u32x2*>(orow + d0) = w;
          }
      }
      if (row < Sq) {
        if (lse != nullptr && g == 0)
          lse[(size_t)bh * Sq + row] =
              lt > 0.0f ? 0.69314718055994531f * (m[0] + __builtin_amdgcn_logf(lt)) : -INFINITY;
      }
    }
  };

  const int n_wg = (int)gridDim.x;
  // XCD-grouped order.  Workgroup i runs on XCD i mod 8 (measured on the
  // device), so the workgroups of an XCD share its L2.  Each XCD takes
  // the kv heads u with u mod 8 = its index, and walks their items head by
  // head (within a head, query blocks heaviest first, the query heads of a
  // GQA group side by side), its workgroup c taking positions c, 2C - 1 - c,
  // 2C + c, ... of that list (C workgroups per XCD).  So all of an XCD's
  // compute units work on the same kv head at the same time and fetch its K/V
  // tiles into one L2 about once, instead of once per round of the global
  // order below; and, as there, a causal workgroup's heavy and light items
  // pair up.  Used when the grid and the kv heads divide into the 8 XCDs,
  // else the global order.
  const int grp_q = Hq / Hkv;  // query heads per kv head
  const int n_kvh = n_bh / grp_q;
  const int C = n_wg >> 3;
  const bool xcd_order =
      ATTN_XCD_ORDER && !PART && (n_wg & 7) == 0 && C > 0 && (n_kvh & 7) == 0;
  const int xcd = (int)blockIdx.x & 7, c_in = (int)blockIdx.x >> 3;
  const int per_xcd = (n_kvh >> 3) * grp_q * n_qt;
  for (int round = 0;; ++round) {
    int sp = 0, bh, qt;
    if (xcd_order) {
      const int p = round * C + ((round & 1) ? C - 1 - c_in : c_in);
      if (p >= per_xcd) break;
      const int ui = p / (grp_q * n_qt);
      const int rem = p - ui * (grp_q * n_qt);
      const int rank = rem / grp_q;
      const int u = xcd + 8 * ui;  // kv head b * Hkv + hkv
      const int bb = u / Hkv;
      bh = bb * Hq + (u - bb * Hkv) * grp_q + (rem - rank * grp_q);
      qt = causal ? (n_qt - 1 - rank) : rank;
    } else {
      const int item =
          round * n_wg + ((round & 1) ? n_wg - 1 - (int)blockIdx.x : (int)blockIdx.x);
      if (item >= n_items) break;
      sp = PART ? item % n_split : 0;
      const int t = PART ? item / n_split : item;
      const int rank = t / n_bh;
      bh = t - rank * n_bh;
      qt = causal ? (n_qt - 1 - rank) : rank;
    }
    const int b = bh / Hq;
    const int hq = bh - b * Hq;
    const int hkv = hq / grp_q;

    // keys [kv0, kv0 + Sk) of the head, indexed from kv0 below
    const int kv0 = PART ? sp * split_keys : 0;
    const int Sk = PART ? max(0, min(Sk_all - kv0, split_keys)) : Sk_all;
    const unsigned char* qh = q + (size_t)bh * Sq * ROW;
    const unsigned char* kh = k + (((size_t)b * Hkv + hkv) * Sk_all + kv0) * ROW;
    const unsigned char* vh = v + (((size_t)b * Hkv + hkv) * Sk_all + kv0) * ROW;
    // key i (from kv0) is visible to row r iff i <= r + causal_off
    const int causal_off = Sk_all - Sq - kv0;

    const int q0 = qt * BR;
    const int qw0 = q0 + wave * 32;  // this wave's first query row

    // keys this workgroup needs
    int kv_end = Sk;
    if (causal) {
      const int last_q = min(q0 + BR, Sq) - 1;
      kv_end = min(Sk, max(0, last_q + causal_off + 1));
    }
    const int n_tiles = (kv_end + KT - 1) / KT;
    // tiles this wave computes: up to its own last visible key, none without rows
    int n_wave = 0;
    if (qw0 < Sq) {
      const int wave_last_q = min(qw0 + 32, Sq) - 1;
      const int wave_kv_end = causal ? min(Sk, max(0, wave_last_q + causal_off + 1)) : Sk;
      n_wave = (wave_kv_end + KT - 1) / KT;
    }

    // Q^T operands of the wave's query n; rows past Sq read as zeros.  Waited
    // for together with the first K tile (and this wave's last stores)
    typename F::QFrag qf;
    if constexpr (F::STAGE_IO) {
      // the wave's 32 rows into its slice, whole rows per instruction
      const __amdgpu_buffer_rsrc_t qr =
          make_rsrc(qh + (size_t)qw0 * ROW, (long long)(Sq - qw0) * ROW);
#pragma unroll
      for (int c = 0; c < 32 * ROW / 1024; ++c)
        load_chunk(qr, F::template load_offset<false>(c), slice_ptr + c * 1024);
    } else {
      const __amdgpu_buffer_rsrc_t qr = make_rsrc(qh, (long long)Sq * ROW);
      F::load_q(qf, qr, (unsigned)((qw0 + n) * ROW));
    }

    // The loading waves split every tile: with L of them, chunk L*c + w covers
    // rows 4(L*c + w) + lane/16 (w = the wave's index among the loaders); L*c*4
    // is a multiple of 16 rows, so one swizzle pattern (and one lane offset)
    // serves all of a wave's chunks
    constexpr int LOADERS = LM >= 2 ? NW : NW / 2;
    constexpr int CHUNKS_PER_LOADER = G::CHUNKS / LOADERS;
    static_assert(CHUNKS_PER_LOADER * LOADERS == G::CHUNKS && (LOADERS * G::RPC) % 16 == 0,
                  "whole chunks per loader, 16-row strides");
    const unsigned koff = F::template load_offset<false>(wave & (LOADERS - 1));
    const unsigned voff = F::template load_offset<true>(wave & (LOADERS - 1));
    unsigned char ATTN_LDS* lds = (unsigned char ATTN_LDS*)(smem);
    // This wave's share of tile j of K or V; keys past Sk read as zeros.
    // HEAD_RSRC: one descriptor per head, covering its Sk keys, and the tile's
    // position in the lanes' offsets (one vector add per load instruction),
    // instead of a descriptor built per tile (some twenty scalar instructions
    // in the phase that issues the loads).  Offsets stay below 2^32: the last
    // tile ends by Sk rounded up to KT keys, at most 2^24 keys of 256 bytes.
    const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(kh, (long long)Sk * ROW);
    const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(vh, (long long)Sk * ROW);
    auto issue = [&](bool is_v, unsigned lane_off, int j, unsigned char ATTN_LDS* dst) {
      const int key0 = j * KT;
      if constexpr (F::HEAD_RSRC) {
        const unsigned toff = (unsigned)key0 * (unsigned)ROW;
#pragma unroll
        for (int c = 0; c < CHUNKS_PER_LOADER; ++c)
          load_chunk(is_v ? v_rs : k_rs, lane_off + (toff + c * LOADERS * 1024),
                     dst + (c * LOADERS + (wave & (LOADERS - 1))) * 1024);
      } else {
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc((is_v ? vh : kh) + (size_t)key0 * ROW, (long long)(Sk - key0) * ROW);
#pragma unroll
        for (int c = 0; c < CHUNKS_PER_LOADER; ++c)
          load_chunk(r, lane_off + c * LOADERS * 1024,
                     dst + (c * LOADERS + (wave & (LOADERS - 1))) * 1024);
      }
    };
    auto stage = [](int j) { return ST == 2 ? (j & 1) : j % ST; };
    auto k_stage = [&](int j) { return lds + stage(j) * TILE_BYTES; };
    auto v_stage = [&](int j) { return lds + (ST + stage(j)) * TILE_BYTES; };
    const LaneAddr la = F::lanes();
    const unsigned lds_base = (unsigned)(size_t)lds;

    f32x16 s[2][QB];
    typename F::PFrag pf;

    // Every wave runs the same sequence  [MFMA(j)] barrier [softmax(j)] barrier,
    // group B one barrier later than group A, so each half-step pairs A's MFMA
    // phase with B's softmax phase and vice versa.  Group A issues K(j+1) and
    // V(j) at the start of its step j and waits for them at its end: their
    // stages were last read by B's MFMA phase of step j-1, which ends before the
    // barrier A passes to start step j, and they are next read by A's MFMA phase
    // of step j+1.
    // The loads of step j, K(j+1) and V(j), are issued at the start of the
    // half-step in which A runs its MFMA phase j, and have landed by the end of
    // the next one.  A issues its share at the start of its MFMA phase and waits
    // at the end of its softmax phase; B issues its share at the start of its
    // softmax phase (of step j-1) and waits at the end of its MFMA phase j.
    // Either way the stages written are free (last read before the barrier that
    // opens the half-step) and are next read after the barrier that closes the
    // wait.  ATTN_LOADERS: 0 = A loads everything, 1 = B does, 2 = both halves
    // (the issue of direct-to-LDS loads holds up the issuing wave for a while,
    // so the cost is best split between the two phases of the half-step).
    // ATTN_LOADERS 3 (with three stages per ring): both groups issue half of
    // step j+1's loads, K(j+2) and V(j+1), at the start of their softmax phase
    // j, and wait for them at the end of their next MFMA phase.  A's softmax
    // phase j runs beside B's MFMA phase j, which reads K(j) and V(j-1); the
    // stages written held K(j-1) and V(j-2), last read in MFMA phase j-1.  So
    // each softmax phase carries half the issue cost, and the DMA writes into
    // LDS land half beside each group's MFMA phase.
    constexpr bool SOFTMAX_LOADS = LM == 3;
    constexpr bool A_LOADS = LM != 1, B_LOADS = LM != 0;
    const bool loader = group_a ? A_LOADS : B_LOADS;
    auto issue_step = [&](int j) {
      if (j + 1 < n_tiles) issue(false, koff, j + 1, k_stage(j + 1));
      if (j < n_tiles) issue(true, voff, j, v_stage(j));
    };
    auto mfma_begin = [&](int j) {
      if (A_LOADS && !SOFTMAX_LOADS && group_a) issue_step(j);
    };
    auto mfma_end = [&]() {
      if (SOFTMAX_LOADS || (B_LOADS && !group_a)) vm_wait_all();
    };
    auto softmax_begin = [&](int j) {
      if (SOFTMAX_LOADS || (B_LOADS && !group_a)) issue_step(j + 1);
    };
    auto softmax_end = [&]() {
      if (A_LOADS && !SOFTMAX_LOADS && group_a) vm_wait_all();
    };
    auto barrier = [] { __builtin_amdgcn_s_barrier(); };
    auto k_addr = [&](int j) { return lds_base + (unsigned)(stage(j) * TILE_BYTES); };
    auto v_addr = [&](int j) { return lds_base + (unsigned)((ST + stage(j)) * TILE_BYTES); };
    float alpha[QB];
    // Tile j crosses the end of the keys or (causal) the diagonal of some row
    // of the wave.  16-bit: j >= mask_from, the first j with (j + 1) KT > Sk or
    // with j KT + KT - 1 > qw0 + causal_off (a floor division by the
    // power-of-two KT, as an arithmetic shift), one compare per step.  FP8
    // keeps the test per tile (the precomputed bound measured -2.6% there).
    int mask_from = Sk >> LOG2_KT;
    if (causal) mask_from = min(mask_from, (qw0 + causal_off + 1) >> LOG2_KT);
    auto masked = [&](int j) {
      if constexpr (F::FP8) {
        const int key0 = j * KT;
        return (key0 + KT > Sk) || (causal && key0 + KT - 1 > qw0 + causal_off);
      } else {
        return j >= mask_from;
      }
    };
    // online softmax of tile j without touching O: returns whether some lane's
    // finite reference max moved, i.e. whether O must still be scaled by alpha
    auto softmax_keep_o = [&](int j) {
      const int key0 = j * KT;
      if (masked(j))
        return softmax_step<DT, QB, true, false>(s, acc, m, l, pf, scale_log2, key0, qw0, Sk,
                                                 causal != 0, causal_off, alpha);
      // the max-free form rests on the threshold rule, which FP8 does not use
      if (ATTN_FAST_SOFTMAX && !F::FP8 && !softmax_fast<DT, QB>(s, m, l, pf, scale_log2))
        return false;
      return softmax_step<DT, QB, false, false>(s, acc, m, l, pf, scale_log2, key0, qw0, Sk,
                                                false, 0, alpha);
    };
    // the same with O scaled by alpha
    auto softmax_scale_o = [&](int j) {
      const int key0 = j * KT;
      if (masked(j))
        softmax_step<DT, QB, true>(s, acc, m, l, pf, scale_log2, key0, qw0, Sk, causal != 0,
                                   causal_off, alpha);
      else
        softmax_step<DT, QB, false>(s, acc, m, l, pf, scale_log2, key0, qw0, Sk, false, 0, alpha);
    };
    auto prio_hi = [] {
      if (ATTN_SETPRIO) __builtin_amdgcn_s_setprio(1);
    };
    auto prio_lo = [] {
      if (ATTN_SETPRIO) __builtin_amdgcn_s_setprio(0);
    };
    // The softmax phase bounds each half-step: the wave in it shares its
    // SIMD's issue cycles with the other group's wave in its MFMA phase, which
    // has a few hundred cycles of slack.  Raising the softmax wave's priority
    // for the phase's vector work gives it those cycles first (measured
    // +0.6% to +0.8% on the 16-bit workloads, bitwise equal).
    auto sm_prio_hi = [] {
      if (F::PRIO_SOFTMAX) __builtin_amdgcn_s_setprio(1);
    };
    auto sm_prio_lo = [] {
      if (F::PRIO_SOFTMAX) __builtin_amdgcn_s_setprio(0);
    };

    if (loader && n_tiles > 0) issue(false, koff, 0, k_stage(0));
    vm_wait_all();
    if constexpr (F::STAGE_IO) {
      unsigned sl = slice;
      asm volatile("" : "+s"(sl));  // as in the epilogue
      F::read_q(qf, sl, la);
    }
    m[0] = -INFINITY;
    l[0] = 0.0f;
#pragma unroll
    for (int db = 0; db < F::DBLOCKS; ++db) acc[db][0] = f32x16{};
    // A's half of step 0 (K(1), V(0)), waited at the end of its first MFMA phase
    if (SOFTMAX_LOADS && group_a) issue_step(0);
    barrier();
    if (!group_a) {
      softmax_begin(-1);  // the half-step before B's first MFMA phase
      barrier();
    }
    // The loop is peeled at this wave's first and last computed tile, and the
    // middle runs in two loops, so that inside each loop the accumulator is
    // updated unconditionally (a path that skips an update makes the register
    // allocator copy the accumulator on every iteration).  The first loop never
    // scales O: with the threshold rule alpha is exactly 1 until some lane's
    // finite reference max moves, which for most rows never happens after their
    // first tile.  When it does, O is scaled once and the rest of the tiles run
    // in the second loop, which scales O on every tile as the recurrence is
    // written.  The first tile needs no scaling: O is still zero.  (With the
    // exact running max of FP8, a wave usually reaches the second loop within
    // its first few tiles.)
    // MFMA phase of step j, 0 < j < n_wave, in the format's order
    auto mfma_phase = [&](int j) {
      if constexpr (F::ORDER == QK_FIRST) {
        F::qk(k_addr(j), la, qf, s);
        F::pv(v_addr(j - 1), la, pf, acc);
      } else {
        F::pv(v_addr(j - 1), la, pf, acc);
        F::qk(k_addr(j), la, qf, s);
      }
    };
    int j = 0;
    if (n_wave > 0) {
      mfma_begin(0);
      prio_hi();
      F::qk(k_addr(0), la, qf, s);
      prio_lo();
      mfma_end();
      barrier();
      softmax_begin(0);
      softmax_keep_o(0);
      softmax_end();
      barrier();
      for (j = 1; j < n_wave; ++j) {
        mfma_begin(j);
        prio_hi();
        mfma_phase(j);
        prio_lo();
        mfma_end();
        barrier();
        softmax_begin(j);
        sm_prio_hi();
        const bool moved = softmax_keep_o(j);
        sm_prio_lo();
        softmax_end();
        barrier();
        if (moved) {
#pragma unroll
          for (int db = 0; db < F::DBLOCKS; ++db) acc[db][0] *= alpha[0];
          ++j;
          break;
        }
      }
      for (; j < n_wave; ++j) {
        mfma_begin(j);
        prio_hi();
        mfma_phase(j);
        prio_lo();
        mfma_end();
        barrier();
        softmax_begin(j);
        sm_prio_hi();
        softmax_scale_o(j);
        sm_prio_lo();
        softmax_end();
        barrier();
      }
      mfma_begin(j);
      prio_hi();
      F::pv(v_addr(j - 1), la, pf, acc);
      prio_lo();
      mfma_end();
      barrier();
      softmax_begin(j);
      epilogue(bh, qw0, sp);
      softmax_end();
      barrier();
      ++j;
    } else {
      epilogue(bh, qw0, sp);  // no key for this wave's rows (or no rows)
    }
    for (; j <= n_tiles; ++j) {  // steps with nothing left for this wave
      mfma_begin(j);
      mfma_end();
      barrier();
      softmax_begin(j);
      softmax_end();
      barrier();
    }
    if (group_a) barrier();

  }
}

// Compute units of the device `stream` runs on (0 if unknown), cached per device.
static int compute_units(hipStream_t stream) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if ((stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) != hipSuccess || dev < 0 ||
      dev >= 64)
    return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <typename F, bool PART>
static void launch_fwd_t(const FwdArgs& a, const FwdSplitArgs* sa, hipStream_t stream) {
  const int n_bh = a.B * a.Hq;
  const int n_qt = (a.Sq + FWD_BR - 1) / FWD_BR;
  const int n_split = PART ? sa->num_splits : 1;
  const long long items = (long long)n_bh * n_qt * n_split;
  const int cus = ATTN_PERSIST ? compute_units(stream) : 0;
  dim3 grid((unsigned)(cus > 0 && items > cus ? cus : items)), block(FWD_NW * 64);
  hipLaunchKernelGGL((fa_fwd_kernel<F, PART>), grid, block, 0, stream,
                     static_cast<const unsigned char*>(a.q), static_cast<const unsigned char*>(a.k),
                     static_cast<const unsigned char*>(a.v), static_cast<uint16_t*>(a.o), a.lse,
                     a.Hq, a.Hkv, a.Sq, a.Sk, a.causal, a.scale_log2, a.o_scale, n_bh, n_qt,
                     PART ? sa->o_part : nullptr, PART ? sa->lse_part : nullptr, n_split,
                     PART ? sa->split_keys : 0, (int)items);
}

template <bool PART>
static hipError_t launch_fwd_any(const FwdArgs& a, const FwdSplitArgs* sa, hipStream_t stream) {
  if (a.fp8)
    a.dtype == 0 ? launch_fwd_t<In8<0>, PART>(a, sa, stream)
                 : launch_fwd_t<In8<1>, PART>(a, sa, stream);
  else if (a.d == 64)
    a.dtype == 0 ? launch_fwd_t<In16<0, 64>, PART>(a, sa, stream)
                 : launch_fwd_t<In16<1, 64>, PART>(a, sa, stream);
  else
    a.dtype == 0 ? launch_fwd_t<In16<0, 128>, PART>(a, sa, stream)
                 : launch_fwd_t<In16<1, 128>, PART>(a, sa, stream);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  return launch_fwd_any<false>(a, nullptr, stream);
}

hipError_t launch_fwd_split(const FwdArgs& a, const FwdSplitArgs& sa, hipStream_t stream) {
  return launch_fwd_any<true>(a, &sa, stream);
}

}  // namespace attn
