// Prefill / extend attention over the paged KV cache (many query rows per
// sequence).  gfx950: MFMA for both contractions, K/V tiles staged in LDS.
//
// What is computed is the scaled dot-product attention of Transformer 추론 커널
// (3/10), §10, in the tiled online-softmax order of §11-§12: per query tile the
// output accumulator, running max and running sum stay on chip while K/V tiles
// stream through; the score matrix never reaches HBM and the result is exact
// (up to rounding).  Keys come through the block table (§14); the query heads
// that share one KV head are served by the same workgroup so each K/V tile is
// loaded once for the whole group (§15).
//
// Layout of the work (one workgroup = NW waves, 4 or 8; a persistent grid
// walks the items, see prefill_kernel):
//  * A wave owns 32 query rows of ONE query head: rows = tokens
//    [wt0, wt0 + 32) of one sequence.  The NW waves are HW heads x TPW token
//    blocks of the same KV head (HW * TPW = NW; HW divides the group size).
//  * Scores are formed transposed, S^T = K . Q^T, with the 32x32 MFMA.  In the
//    accumulator layout every lane then holds ONE query row (lane % 32) and 16
//    of the 32 keys of a block, so row max / row sum are in-lane plus a single
//    exchange with lane ^ 32, and the probabilities P are already laid out as
//    the B operand of O^T = V^T . P^T -- no shuffle between the two MFMAs.
//  * bf16: V is written to LDS transposed (d-major) so the A operand of the PV
//    MFMA (8 keys of one d per lane) is two 8-byte LDS reads.  fp32: the 32x32x2
//    MFMA takes one element per lane, so V stays row-major.
//  * K/V tiles are double-buffered in LDS; the next tile's global loads are
//    issued before the current tile's math.  Rows past the last key an item
//    needs are never trusted: V is zeroed there and K scores are masked, and
//    table entries past a sequence's last block are never used.
//  * Causal (bottom-right, with cached prefix c = Lk - Lq): tiles wholly above
//    a wave's rows are skipped; only tiles crossing the diagonal are masked.
//  * FP8 caches (the KV8 instantiations, bf16 queries): each lane loads the
//    8 codes behind the 16-byte chunk the bf16 copy would have moved (same
//    element offsets: one code per element) and the scale of its key row,
//    dequantizes them to bf16 in registers and writes them to the same LDS
//    place after the step's math; the rest of the kernel is the bf16 one.
//  * Sliding window W (the WIN instantiations): the row at position p sees
//    keys p - W + 1 .. p.  An item's key tiles start at the tile holding its
//    first row's window start; rows before that start are copied as zero rows
//    (their table entries are never read), tiles wholly below a wave's
//    windows are skipped, and tiles crossing a window's lower edge are masked.
#pragma once
#include <type_traits>

#include "kvs_device.hpp"
#include "kvs_internal.hpp"

namespace kvs {

// Largest growth (base 2) of a row maximum absorbed without rescaling.
constexpr float kRescaleSlack = 8.0f;

template <int D, bool BF16, int NW = 4>
struct PCfg {
  static constexpr int NTH = 64 * NW;          // threads per workgroup
  static constexpr int BN = BF16 ? 64 : 32;   // keys per tile
  static constexpr int ESZ = BF16 ? 2 : 4;    // element bytes
  // bf16: K and V tiles are row-major without padding, filled by 16-byte
  // global-to-LDS copies; the 16-byte chunks of a row are XOR-swizzled by key
  // so that the lanes of one LDS read hit distinct banks: a score-operand
  // read (16 bytes per lane, 16 lanes a cycle) takes 16 different chunks of
  // 16 rows; a transposing V read (8 bytes per lane, 32 lanes a cycle) takes
  // 4 chunks of each of 4 rows, which the V swizzle moves to 16 different
  // chunks (rows are 64 banks wide at D = 128, so without it the 4 rows would
  // share 32 banks).  fp32: padded rows written from registers.
  static constexpr int KROW = BF16 ? D * 2 : D * 4 + 16;   // bytes per K row in LDS
  static constexpr int VROW = BF16 ? D * 2 : D * 4 + 16;   // bytes per V row in LDS
  static constexpr int KTILE = BN * KROW;
  static constexpr int VTILE = BN * VROW;
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int NPG = BN / 16;          // pages per tile
  static constexpr int CPR = D * ESZ / 16;     // 16-byte chunks per token row
  static constexpr int KCH = BN * CPR;         // chunks per tile and operand
  static constexpr int KIT = (KCH + NTH - 1) / NTH;  // chunks per thread and operand
  static constexpr int KPW = 64 * KIT / CPR;   // bf16: key rows each wave copies
  static constexpr int NDB = D / 32;           // 32-wide d blocks of the output
  // bf16 chunk slot of logical chunk c of key row `key`: c ^ swizzle(key)
  __host__ __device__ static constexpr int kswz(int key) { return D == 128 ? (key & 15) : ((key >> 1) & 7); }
  __host__ __device__ static constexpr int vswz(int key) { return D == 128 ? ((key & 3) << 2) : ((key & 2) << 1); }
};
static_assert(PCfg<128, true>::STAGE == 32768 && PCfg<64, true>::STAGE == 16384 &&
                  PCfg<128, false>::STAGE == 2 * 32 * (128 * 4 + 16),
              "the host's prefill_stage_bytes must match the stage layout");
template <int D, int NW>
constexpr bool copies_whole_pages() {
  using C = PCfg<D, true, NW>;
  return C::KIT * C::NTH == C::KCH && C::KPW * C::CPR == 64 * C::KIT && 16 % C::KPW == 0;
}
static_assert(copies_whole_pages<128, 4>() && copies_whole_pages<64, 4>() && copies_whole_pages<128, 8>() &&
                  copies_whole_pages<64, 8>(),
              "bf16: each wave copies KIT whole 1 KiB blocks: KPW consecutive keys of one page of a tile");

// Source of the key rows past an item's last key: a zero row, so V is exactly
// 0 there (P is 0 too, but V could hold anything) and K is harmless.
static __device__ __attribute__((aligned(16))) uint16_t g_zero_row[128];

// Persistent work loop, two workgroups per CU (two waves per SIMD): one
// workgroup's barrier and load waits overlap the other's math.
//
// An item is (sequence b, token tile of TW rows, head group); items are
// enumerated tile-major from the last token tile down, so under a causal mask
// the heaviest items come first, and dealt to the workgroups in snake order
// (round r: workgroup w takes item r*G + w, in odd rounds the mirror image of
// w among the workgroups of its XCD), which evens out the work.  A workgroup walks its items as ONE stream of
// (item, key tile) steps: the next step's K/V loads -- also the first tile of
// the next item -- are issued before the current step's math, block-table
// entries one step earlier, and the next item's Q rows as soon as the last
// score tile of the current item is formed, so moving to a new item costs
// about what moving to a new key tile does.
// 8 E4M3 codes times a scale, rounded to bf16 (nearest even): one 16-byte
// chunk of a bf16 row.  The conversion instruction decodes the OCP E4M3
// format exactly.
__device__ __forceinline__ u32x4 e4m3x8_scaled_to_bf16(const u32x2& w, float sc);
// 8 INT8 codes times a scale, rounded to bf16 (nearest even): each code is
// its sign-extended byte, converted exactly to fp32.
__device__ __forceinline__ u32x4 i8x8_scaled_to_bf16(const u32x2& w, float sc) {
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t u = w[h];
    r[2 * h] = pack_bf16x2((float)(int8_t)(u & 0xFFu) * sc, (float)(int8_t)((u >> 8) & 0xFFu) * sc);
    r[2 * h + 1] = pack_bf16x2((float)(int8_t)((u >> 16) & 0xFFu) * sc, (float)(int8_t)(u >> 24) * sc);
  }
  return r;
}
template <bool I8>
__device__ __forceinline__ u32x4 q8x8_scaled_to_bf16(const u32x2& w, float sc) {
  if constexpr (I8) return i8x8_scaled_to_bf16(w, sc);
  else return e4m3x8_scaled_to_bf16(w, sc);
}
__device__ __forceinline__ u32x4 e4m3x8_scaled_to_bf16(const u32x2& w, float sc) {
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const auto f = (h & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(w[h >> 1], true)
                           : __builtin_amdgcn_cvt_pk_f32_fp8(w[h >> 1], false);
    r[h] = pack_bf16x2(f[0] * sc, f[1] * sc);
  }
  return r;
}

// I8: the KV8 caches hold INT8 codes, not E4M3.
// The workgroup's part of the persistent loop: workgroup w of G.  pre_nt >= 0:
// the caller has already staged the batch metadata below (same LDS place) and
// found the most token tiles of any sequence, pre_nt.
template <int D, bool BF16, int NW, bool WIN, bool KV8, bool I8 = false>
__device__ __forceinline__ void prefill_body(AttnParams p, const int G, const int w, const int pre_nt = -1) {
  static_assert(!KV8 || BF16, "FP8 / INT8 caches take bf16 queries");
  static_assert(!I8 || KV8, "INT8 codes are a KV8 cache");
  using C = PCfg<D, BF16, NW>;
  using E = typename std::conditional<BF16, uint16_t, float>::type;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int s_nt[NW];

  const int tid = threadIdx.x;
  // wave-uniform by construction; readfirstlane lets the compiler see it, so
  // every per-wave decision below is a scalar branch
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int B = p.B;
  const int TW = 32 * p.TPW;
  const int tw_shift = 5 + __builtin_ctz(p.TPW);   // log2(TW): TPW is a power of two
  const int hw = wave % p.HW, tb = wave / p.HW;
  const int64_t kv_tok_stride = (int64_t)p.Hkv * D;   // elements between token rows
  const int64_t page_stride = (int64_t)kPage * kv_tok_stride;   // elements per block

  // ---- batch metadata: cu_seqlens_q and seqlens_k staged in LDS (when the
  // planner has room for them), and the most token tiles of any sequence ----
  const bool staged = p.meta_lds != 0;
  int* s_cq = reinterpret_cast<int*>(smem + 2 * C::STAGE);   // [B + 1]
  int* s_lk = s_cq + B + 1;                                   // [B]
  if (pre_nt < 0) {
    float ntmax = 0.f;
    for (int b = tid; b < B; b += C::NTH) {
      const int a = p.cu_q[b], z = p.cu_q[b + 1], lk = p.lens_k[b];
      if (staged) {
        s_cq[b] = a;
        s_lk[b] = lk;
        if (b == B - 1) s_cq[B] = z;
      }
      ntmax = fmaxf(ntmax, (float)((z - a + TW - 1) >> tw_shift));
    }
    ntmax = wave_max(ntmax);
    if (lane == 0) s_nt[wave] = (int)ntmax;
    __syncthreads();
  }
  int nt_all = pre_nt;
  if (pre_nt < 0) {
    nt_all = s_nt[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) nt_all = max(nt_all, s_nt[i]);
  }
  const int NT = __builtin_amdgcn_readfirstlane(nt_all);
  const int64_t BH = (int64_t)B * p.NHG;
  const int64_t NI = (int64_t)NT * BH;
  const int rev_w = (G & 7) == 0 ? (w & 7) + 8 * (G / 8 - 1 - (w >> 3)) : G - 1 - w;
  // Item order.  A pair (sequence, head group) -- whose token tiles all read
  // the same keys -- belongs to one XCD (pair % 8; workgroup w runs on XCD
  // w % 8), and each XCD's workgroups take its pairs a few at a time, all
  // token tiles of a pair in one round, heaviest (last) tile first; odd
  // rounds run the other way round, so each workgroup's causal work evens out.
  // The K/V a round re-reads then fits the XCD's L2.  (items32 = 0: the same
  // tile-major order over all workgroups with 64-bit indices.)
  const int X = (G & 7) == 0 ? 8 : 1;
  const int xcd = w % X, wi = w / X, GX = G / X;
  const int NPx = (int)((BH - xcd + X - 1) / X);   // pairs of this XCD
  const int64_t NIx = (int64_t)NPx * NT;           // its items
  const int64_t nrounds = p.items32 ? (NIx + GX - 1) / GX : (NI + G - 1) / G;
  // NT < 2^31: q = v / NT by multiply-high (see fast_div_magic)
  uint32_t nt_l = 0;
  while ((1u << nt_l) < (uint32_t)NT && nt_l < 31) ++nt_l;
  const uint32_t nt_m = (uint32_t)((((uint64_t)1) << (32 + nt_l)) / (uint32_t)max(NT, 1) - (((uint64_t)1) << 32) + 1);

  // ---- heaviest items first (up to 256 sequences of unequal shapes) -------
  // The order above hands every workgroup the same number of items, which
  // balances the work when the sequences are alike.  When they differ (an
  // extend batch: prompts and cached prefixes of many lengths) it does not:
  // rounds pass over tiles a shorter sequence lacks, and a round takes a few
  // workgroups to items many times heavier than the rest.  Then this XCD's
  // items are ranked by decreasing key tiles (ties: sequence, head group,
  // token tile from the last) and dealt in the same snake order.  Lane l
  // holds sequences l, l + 64, ..., and A(c), the number of items of c or
  // more key tiles, is a wave sum of closed forms, so the item of rank v is
  // found by a binary search over c and a prefix sum over the sequences of
  // level c.  Each wave finds every NW-th round's item; the list sits in LDS.
  // (With a window an item's key tiles start at its window's first one.)
  int* s_pair = s_lk + B;                 // [kSortRounds] pair b * NHG + hgrp of round r, -1: none
  int* s_tile = s_pair + kSortRounds;     // [kSortRounds] its token tile
  bool sorted = false;
  int nrounds_s = 0;
  if (staged && p.items32 && B <= kSortB) {
    constexpr int SQ = kSortB / 64;   // sequences per lane: lane + 64 q
    const int nq = (B + 63) >> 6;      // blocks of 64 sequences in use
    int sLq[SQ], sCached[SQ], sNT[SQ], sMult[SQ], sH0[SQ], sLk[SQ];
    const float big = 3.0e9f;
    float lq_lo = big, lq_hi = -big, c_lo = big, c_hi = -big, kmaxf = 0.f;
#pragma unroll
    for (int q = 0; q < SQ; ++q) {
      const int b = 64 * q + lane;
      sLq[q] = sCached[q] = sNT[q] = sMult[q] = sH0[q] = sLk[q] = 0;
      if (b < B) {
        sLk[q] = s_lk[b];
        sLq[q] = s_cq[b + 1] - s_cq[b];
        sCached[q] = sLk[q] - sLq[q];
        sNT[q] = (p.mixed && sLq[q] == 1) ? 0 : (sLq[q] + TW - 1) >> tw_shift;
        sH0[q] = ((xcd - (b * p.NHG) % X) % X + X) % X;   // first head group of sequence b on this XCD
        sMult[q] = (sNT[q] > 0 && sH0[q] < p.NHG) ? (p.NHG - 1 - sH0[q]) / X + 1 : 0;
      }
      if (sNT[q] > 0) {
        lq_lo = fminf(lq_lo, (float)sLq[q]);
        lq_hi = fmaxf(lq_hi, (float)sLq[q]);
        c_lo = fminf(c_lo, (float)sCached[q]);
        c_hi = fmaxf(c_hi, (float)sCached[q]);
        kmaxf = fmaxf(kmaxf, (float)((sLk[q] + C::BN - 1) / C::BN));
      }
    }
    // the same shape for every sequence with items: the order above is as good
    lq_lo = -wave_max(-lq_lo);
    lq_hi = wave_max(lq_hi);
    c_lo = -wave_max(-c_lo);
    c_hi = wave_max(c_hi);
    // a window: an item spans at most ceil((W + TW - 1) / BN) + 1 key tiles,
    // so the cost is taken as min(key tiles, that): still non-decreasing over
    // a sequence's token tiles, and the items at the cap rank as equals
    const int wcap = WIN ? (int)min(((int64_t)p.window + TW - 1 + C::BN - 1) / C::BN + 1, (int64_t)0x7fffffff)
                         : 0x7fffffff;
    const int kmax = min((int)wave_max(kmaxf), wcap);
    // first token tile of sequence 64 q + lane whose items see more than (c - 1) * BN keys
    auto first_tile = [&](int q, int c) __attribute__((always_inline)) {
      if (c > wcap) return sNT[q];   // past the cap: no item
      const int keys = C::BN * (c - 1);
      if (!p.causal) return sLk[q] > keys ? 0 : sNT[q];
      const int need = keys - sCached[q] + 1;   // rows the item must reach
      return need > sLq[q] ? sNT[q] : (need <= 0 ? 0 : ((need + TW - 1) >> tw_shift) - 1);
    };
    auto wave_total = [&](int x) __attribute__((always_inline)) {
      return __builtin_amdgcn_readlane(wave_inclusive_sum(x), 63);
    };
    auto items_from_level = [&](int c) __attribute__((always_inline)) {
      int x = 0;
#pragma unroll
      for (int q = 0; q < SQ; ++q)
        if (q < nq) x += sMult[q] * (sNT[q] - first_tile(q, c));
      return wave_total(x);
    };
    const int nx = items_from_level(1);
    nrounds_s = (nx + GX - 1) / GX;
    sorted = (lq_lo != lq_hi || c_lo != c_hi) && nrounds_s <= kSortRounds;
    if (sorted) {
      for (int r = wave; r < nrounds_s; r += NW) {
        const int v = r * GX + ((r & 1) ? GX - 1 - wi : wi);
        int pair = -1, tile = 0;
        if (v < nx) {
          int lo = 1, hi = kmax + 1;   // items_from_level(lo) > v >= items_from_level(hi)
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (items_from_level(mid) > v) lo = mid;
            else hi = mid;
          }
          int o = v - items_from_level(lo + 1);   // rank within level lo, counted over the blocks in order
#pragma unroll
          for (int q = 0; q < SQ; ++q) {
            if (q >= nq || pair >= 0) continue;
            const int f1 = first_tile(q, lo + 1), nb = f1 - first_tile(q, lo);
            const int cnt = sMult[q] * nb;
            const int incl = wave_inclusive_sum(cnt);
            const int tot = __builtin_amdgcn_readlane(incl, 63);
            if (o >= tot) {
              o -= tot;
              continue;
            }
            const uint64_t hit = __ballot(cnt > 0 && incl - cnt <= o && o < incl);   // one lane, as 0 <= o < tot
            if (hit != 0) {
              const int L = (int)__builtin_ctzll(hit);   // sequence 64 q + L holds it
              const int j = o - (__builtin_amdgcn_readlane(incl, L) - __builtin_amdgcn_readlane(cnt, L));
              const int nbL = __builtin_amdgcn_readlane(nb, L);
              pair = (64 * q + L) * p.NHG + __builtin_amdgcn_readlane(sH0[q], L) + (j / nbL) * X;
              tile = __builtin_amdgcn_readlane(f1, L) - 1 - j % nbL;
            }
            o = -1;   // found (or, impossibly, no lane: none)
          }
        }
        if (lane == 0) {
          s_pair[r] = pair;
          s_tile[r] = tile;
        }
      }
      __syncthreads();
    }
  }
  sorted = __builtin_amdgcn_readfirstlane((int)sorted) != 0;
  const int64_t nrounds_all = sorted ? nrounds_s : nrounds;

  // ---- items --------------------------------------------------------------
  struct Item {
    int r;             // round of this workgroup's item sequence (nrounds: none)
    int b, hgrp, tile;
    int kvh;           // KV head of the head group
    int q0, Lq, Lk;
    int nkeys, ntiles, npages;
    int klo, t0;       // first key any row of the item sees, its key tile (0 without a window)
  };
  auto meta = [&](int b, int& q0, int& q1, int& lk) __attribute__((always_inline)) {
    // uniform values: readfirstlane keeps the item state in scalar registers
    if (staged) {
      q0 = __builtin_amdgcn_readfirstlane(s_cq[b]);
      q1 = __builtin_amdgcn_readfirstlane(s_cq[b + 1]);
      lk = __builtin_amdgcn_readfirstlane(s_lk[b]);
    } else {
      q0 = __builtin_amdgcn_readfirstlane(p.cu_q[b]);
      q1 = __builtin_amdgcn_readfirstlane(p.cu_q[b + 1]);
      lk = __builtin_amdgcn_readfirstlane(p.lens_k[b]);
    }
  };
  // first non-empty item of round r or later
  auto item_from = [&](int r) __attribute__((always_inline)) {
    Item it;
    it.ntiles = 0;
    for (; r < nrounds_all; ++r) {
      int tile, b, hgrp;
      if (sorted) {
        const int pair = __builtin_amdgcn_readfirstlane(s_pair[r]);
        if (pair < 0) continue;
        tile = __builtin_amdgcn_readfirstlane(s_tile[r]);
        const uint32_t bq = (__umulhi((uint32_t)pair, p.nhg_m) + (uint32_t)pair) >> p.nhg_l;
        b = (int)bq;
        hgrp = pair - (int)bq * p.NHG;
      } else if (p.items32) {
        // this XCD's item v (< 2^31): local pair v / NT, tile counted down
        const int64_t v64 = (int64_t)r * GX + ((r & 1) ? GX - 1 - wi : wi);
        if (v64 >= NIx) continue;
        const uint32_t v = (uint32_t)v64;
        const uint32_t lp = (__umulhi(v, nt_m) + v) >> nt_l;
        tile = NT - 1 - (int)(v - lp * (uint32_t)NT);
        const uint32_t pair = (uint32_t)xcd + (uint32_t)X * lp;
        const uint32_t bq = (__umulhi(pair, p.nhg_m) + pair) >> p.nhg_l;
        b = (int)bq;
        hgrp = (int)(pair - bq * (uint32_t)p.NHG);
      } else {
        // tile-major over all workgroups; odd rounds mirror the workgroups
        // within each XCD, so a pair still stays on one XCD
        const int64_t u = (int64_t)r * G + ((r & 1) ? rev_w : w);
        if (u >= NI) continue;
        const int64_t pair = u % BH;
        tile = NT - 1 - (int)(u / BH);
        b = (int)(pair / p.NHG);
        hgrp = (int)(pair % p.NHG);
      }
      int q0, q1, lk;
      meta(b, q0, q1, lk);
      const int Lq = q1 - q0;
      if (tile * TW >= Lq) continue;   // this sequence has fewer token tiles
      if (p.mixed && Lq == 1) continue;   // a mixed launch's decode part serves one-row sequences
      const int cached = lk - Lq;
      const int tlast = min(tile * TW + TW, Lq) - 1;
      it.b = b;
      it.hgrp = hgrp;
      it.kvh = __builtin_amdgcn_readfirstlane((hgrp * p.HW) / p.G);   // HW divides G: one KV head per item
      it.tile = tile;
      it.q0 = q0;
      it.Lq = Lq;
      it.Lk = lk;
      it.nkeys = p.causal ? min(lk, cached + tlast + 1) : lk;
      it.ntiles = (it.nkeys + C::BN - 1) / C::BN;
      it.npages = (it.nkeys + 15) >> 4;
      it.klo = WIN ? max(0, cached + tile * TW - p.window + 1) : 0;
      it.t0 = it.klo / C::BN;
      break;
    }
    it.r = r;
    return it;
  };
  // a step of the stream: key tile t of item it (it.ntiles == 0: none)
  struct Step {
    Item it;
    int t;
  };
  auto advance = [&](const Step& s) __attribute__((always_inline)) {
    Step x = s;
    if (s.it.ntiles == 0) return x;
    if (s.t + 1 < s.it.ntiles) {
      x.t = s.t + 1;
    } else {
      x.it = item_from(s.it.r + 1);
      x.t = x.it.t0;
    }
    return x;
  };
  auto kv_base = [&](const Item& it, const void* base) __attribute__((always_inline)) {
    return static_cast<const E*>(base) + (int64_t)it.kvh * D;
  };

  // ---- staging helpers ----------------------------------------------------
  // Block-table entries of step s: lane i holds entry t * NPG + (i % NPG)
  // (index clamped to the item's first page -- the one holding klo -- and to
  // the sequence's last page; issue_loads replaces entries past it by block
  // 0).  A vector load, so waiting for it is counted with the other global
  // loads and never holds up an LDS read.
  auto load_pages = [&](const Step& s) -> int {
    if (s.it.ntiles == 0) return 0;
    const int32_t* trow = p.table + (int64_t)s.it.b * p.MB;
    int e = s.t * C::NPG + (lane & (C::NPG - 1));
    if constexpr (WIN) e = max(e, s.it.klo >> 4);
    return trow[min(e, s.it.npages - 1)];
  };
  // Chunk it of a K row-major tile: key row j = (it * NTH + tid) / CPR of the
  // tile (its page index is the same across a wave), 16-byte chunk ch.
  auto kpage_idx = [&](int it) -> int {
    return __builtin_amdgcn_readfirstlane(((it * C::NTH + tid) / C::CPR) >> 4);
  };
  // fp32 path: chunk it of a row-major tile (key row (it * NTH + tid) / CPR)
  // is loaded into registers and written to padded LDS rows; per-lane element
  // offsets inside a block (< 16 * Hkv * D, so 32 bits)
  uint32_t koff[C::KIT];
#pragma unroll
  for (int it = 0; it < C::KIT; ++it) {
    const int cch = it * C::NTH + tid;
    const int j = (cch / C::CPR) & (C::BN - 1), ch = cch % C::CPR;
    koff[it] = (uint32_t)((j & 15) * (int)kv_tok_stride + ch * (16 / C::ESZ));
  }
  u32x4 kreg[BF16 ? 1 : C::KIT];
  u32x4 vreg[BF16 ? 1 : C::KIT];
  // KV8: codes (8 per chunk) and the scale of the chunk's key row
  u32x2 k8[KV8 ? C::KIT : 1], v8[KV8 ? C::KIT : 1];
  float ks8[KV8 ? C::KIT : 1], vs8[KV8 ? C::KIT : 1];
  // bf16: wave w copies keys [w KPW, w KPW + KPW) of every tile, all in page
  // w KPW / 16.  Per lane and copy j, the element offset inside that page of
  // its 16-byte chunk, with the chunk slot swizzled by key: the same for
  // every step.
  uint32_t kpo[BF16 ? C::KIT : 1], vpo[BF16 ? C::KIT : 1];
  if constexpr (BF16) {
#pragma unroll
    for (int j = 0; j < C::KIT; ++j) {
      const int pch = j * 64 + lane;            // chunk of the wave's keys
      const int slot = pch % C::CPR;
      const int key = wave * C::KPW + pch / C::CPR;   // key row in the tile
      // byte offsets for bf16 rows, element (= code byte) offsets for FP8 / INT8
      kpo[j] = (uint32_t)((key & 15) * (int)kv_tok_stride + (slot ^ C::kswz(key)) * 8) * (KV8 ? 1u : 2u);
      vpo[j] = (uint32_t)((key & 15) * (int)kv_tok_stride + (slot ^ C::vswz(key)) * 8) * (KV8 ? 1u : 2u);
    }
  }
  // K/V of step s: bf16 -> 16-byte global-to-LDS copies straight into stage
  // `buf` (each wave writes KIT whole 1 KiB blocks of each tile; key rows at
  // or past nkeys, or before klo, copy the zero row); fp32 -> registers, see
  // write_stage.
  // Raw addresses stay readable: a row past nkeys lies in an owned block or,
  // past the last owned page, in block 0.
  auto issue_loads = [&](int pgv, const Step& s, int buf) {
    const E* kbase = kv_base(s.it, p.k);
    const E* vbase = kv_base(s.it, p.v);
    if constexpr (KV8) {
      // codes and scales into registers; write_stage dequantizes them into LDS
      const int pgi = (wave * C::KPW) >> 4;
      const int pk = s.t * C::NPG + pgi < s.it.npages ? __builtin_amdgcn_readlane(pgv, pgi) : 0;
      const uint8_t* kpage = static_cast<const uint8_t*>(p.k) + (int64_t)s.it.kvh * D + pk * page_stride;
      const uint8_t* vpage = static_cast<const uint8_t*>(p.v) + (int64_t)s.it.kvh * D + pk * page_stride;
      const int64_t so = ((int64_t)pk * p.Hkv + s.it.kvh) * kPage;   // scales [NB, Hkv, 16]
#pragma unroll
      for (int j = 0; j < C::KIT; ++j) {
        const int key = wave * C::KPW + (j * 64 + lane) / C::CPR;   // key row in the tile
        k8[j] = *reinterpret_cast<const u32x2*>(kpage + kpo[j]);
        v8[j] = *reinterpret_cast<const u32x2*>(vpage + vpo[j]);
        ks8[j] = p.k_scale[so + (key & 15)];
        vs8[j] = p.v_scale[so + (key & 15)];
      }
    } else if constexpr (BF16) {
      char* Kd = smem + buf * C::STAGE;
      char* Vd = Kd + C::KTILE;
      // this wave's page of the tile (block 0 past the sequence's last page)
      const int pgi = (wave * C::KPW) >> 4;
      const int pk = s.t * C::NPG + pgi < s.it.npages ? __builtin_amdgcn_readlane(pgv, pgi) : 0;
      // the page's base is wave-uniform and each lane adds a fixed 32-bit
      // byte offset (the scalar-base form of the copy: no per-lane 64-bit
      // address arithmetic)
      const char* kpage = reinterpret_cast<const char*>(kbase + pk * page_stride);
      const char* vpage = reinterpret_cast<const char*>(vbase + pk * page_stride);
      const int kv0 = s.t * C::BN;
      // keys at or past nkeys (only in an item's last tile) and keys before
      // klo (only in its first tiles) copy the zero row
      bool edge = kv0 + wave * C::KPW + C::KPW > s.it.nkeys;   // uniform
      if constexpr (WIN) edge = edge || kv0 + wave * C::KPW < s.it.klo;
      if (!edge) {
#pragma unroll
        for (int j = 0; j < C::KIT; ++j) {
          const int blk = wave * C::KIT + j;   // 1 KiB block of each tile
          // (the empty asm keeps each offset a 32-bit value next to its use, so
          // the copy takes the scalar-base form)
          uint32_t ko = kpo[j], vo = vpo[j];
          asm volatile("" : "+v"(ko), "+v"(vo));
          copy16_to_lds(kpage + ko, Kd + blk * 1024);
          copy16_to_lds(vpage + vo, Vd + blk * 1024);
        }
        __builtin_amdgcn_sched_barrier(0);   // (keeps this path's copies apart from the edge path's)
      } else {
        const char* zero = reinterpret_cast<const char*>(g_zero_row);
#pragma unroll
        for (int j = 0; j < C::KIT; ++j) {
          const int blk = wave * C::KIT + j;
          const int key = wave * C::KPW + (j * 64 + lane) / C::CPR;
          const bool live = kv0 + key < s.it.nkeys && (!WIN || kv0 + key >= s.it.klo);
          const int slot = (j * 64 + lane) % C::CPR;
          const char* ks = live ? kpage + kpo[j] : zero + (slot ^ C::kswz(key)) * 16;
          const char* vs = live ? vpage + vpo[j] : zero + (slot ^ C::vswz(key)) * 16;
          copy16_to_lds(ks, Kd + blk * 1024);
          copy16_to_lds(vs, Vd + blk * 1024);
        }
      }
    } else {
      int pg[C::NPG];
#pragma unroll
      for (int i = 0; i < C::NPG; ++i) {
        const int e = __builtin_amdgcn_readlane(pgv, i);
        pg[i] = s.t * C::NPG + i < s.it.npages ? e : 0;
      }
#pragma unroll
      for (int it = 0; it < C::KIT; ++it) {
        const int pi = kpage_idx(it);
        int pk = pg[0];
#pragma unroll
        for (int i = 1; i < C::NPG; ++i) pk = pi == i ? pg[i] : pk;   // uniform
        kreg[it] = ld16(kbase + pk * page_stride + koff[it]);
        vreg[it] = ld16(vbase + pk * page_stride + koff[it]);
      }
    }
  };
  // fp32: writes step s's registers to LDS buffer `buf`.  V rows at or past
  // nkeys, or before klo, are zeroed (only an item's last or first tiles have
  // any): P is 0 there but V may hold anything.  K rows there stay as loaded:
  // tiles that have them always take the masked path, which selects their
  // scores away.
  auto write_stage = [&](int buf, const Step& s) {
    if constexpr (KV8) {
      // the places the bf16 copies would have written: block wave KIT + j,
      // 16 bytes per lane; keys past nkeys or before klo are zero
      char* Kd = smem + buf * C::STAGE;
      char* Vd = Kd + C::KTILE;
      const int kv0 = s.t * C::BN;
      bool edge = kv0 + wave * C::KPW + C::KPW > s.it.nkeys;   // uniform
      if constexpr (WIN) edge = edge || kv0 + wave * C::KPW < s.it.klo;
      const u32x4 zero = {0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < C::KIT; ++j) {
        const int blk = wave * C::KIT + j;
        const int key = kv0 + wave * C::KPW + (j * 64 + lane) / C::CPR;
        const bool live = !edge || (key < s.it.nkeys && (!WIN || key >= s.it.klo));
        st16(Kd + blk * 1024 + lane * 16, live ? q8x8_scaled_to_bf16<I8>(k8[j], ks8[j]) : zero);
        st16(Vd + blk * 1024 + lane * 16, live ? q8x8_scaled_to_bf16<I8>(v8[j], vs8[j]) : zero);
      }
    } else if constexpr (!BF16) {
      char* Ks = smem + buf * C::STAGE;
      char* Vs = Ks + C::KTILE;
      const int kv0 = s.t * C::BN;
      bool edge = kv0 + C::BN > s.it.nkeys;
      if constexpr (WIN) edge = edge || kv0 < s.it.klo;
      const u32x4 zero = {0, 0, 0, 0};
#pragma unroll
      for (int it = 0; it < C::KIT; ++it) {
        const int cch = it * C::NTH + tid;
        if (cch < C::KCH) {
          const int key = kv0 + cch / C::CPR;
          const bool keep = !edge || (key < s.it.nkeys && (!WIN || key >= s.it.klo));
          st16(Ks + (cch / C::CPR) * C::KROW + (cch % C::CPR) * 16, kreg[it]);
          st16(Vs + (cch / C::CPR) * C::VROW + (cch % C::CPR) * 16, keep ? vreg[it] : zero);
        }
      }
    }
  };
  // bf16 transposing V reads: lane (16-lane group g16, i = lane % 16) reads
  // the 8-byte row of key  base + 4 * (g16 / 2) + i / 4  and d  32 db +
  // 16 (g16 % 2) + 4 (i % 4); the group then holds V^T for 16 d x 4 keys.
  // The key base is a multiple of 4, so the row's swizzle depends on i / 4
  // (each of the 4 rows a 16-lane group reads lands in its own quarter of the
  // 64 banks).
  const int tr_i = lane & 15, tr_g = lane >> 4;
  const int tr_row = (4 * (tr_g >> 1) + (tr_i >> 2)) * C::VROW + (tr_i & 1) * 8;
  const int tr_c = 2 * (tr_g & 1) + ((tr_i & 3) >> 1), tr_sw = C::vswz(tr_i >> 2);

  // ---- Q fragment (B operand of S^T = K . Q^T) of an item ----------------
  // bf16 32x32x16: lane holds Q[row n][ks*16 + hh*8 .. +8] for k-step ks.
  // fp32 32x32x2: lane holds Q[row n][hh*D/2 + ks] for k-step ks.
  // The sign of the scale is moved into Q (an exact sign flip), so the score
  // multiplier c is >= 0 and a row maximum of raw scores is also the maximum of
  // the scaled ones.
  constexpr int QF = BF16 ? D / 16 : D / 2;
  typename std::conditional<BF16, u32x4, float>::type qf[QF];
  const float c = fabsf(p.scale_log2);
  const uint32_t flip = p.scale_log2 < 0.f ? 0x80008000u : 0u;
  auto load_q = [&](const Item& it) __attribute__((always_inline)) {
    const int qrow = it.tile * TW + tb * 32 + n;
    const bool ok = qrow < it.Lq;
    const int h = it.hgrp * p.HW + hw;
    const E* qp = static_cast<const E*>(p.q) + ((int64_t)(it.q0 + (ok ? qrow : 0)) * p.Hq + h) * D;
    // the sign flip is a separate (uniform) step so a prefetch of Q is not
    // waited for where it is issued
    if constexpr (BF16) {
#pragma unroll
      for (int ks = 0; ks < QF; ++ks) qf[ks] = ld16(qp + ks * 16 + hh * 8);   // row clamped to the item's first if !ok
      if (flip) {
#pragma unroll
        for (int ks = 0; ks < QF; ++ks) qf[ks] = u32x4{qf[ks][0] ^ flip, qf[ks][1] ^ flip, qf[ks][2] ^ flip, qf[ks][3] ^ flip};
      }
    } else {
#pragma unroll
      for (int c4 = 0; c4 < QF / 4; ++c4) {
        const u32x4 wq = ld16(qp + hh * (D / 2) + c4 * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[c4 * 4 + e] = __uint_as_float(wq[e]);
      }
      if (flip) {
#pragma unroll
        for (int e = 0; e < QF; ++e) qf[e] = -qf[e];
      }
    }
  };

  // ---- online-softmax state -------------------------------------------
  // m_run is the reference maximum that P and l are taken against (base-2
  // units, same in both lane halves).  It is only moved up when a tile's
  // maximum exceeds it by more than kRescaleSlack: until then P <= 2^slack, and
  // since l and O use the same reference the quotient O / l is unchanged, so
  // most tiles skip rescaling the output accumulators.
  float m_run = kMaskedScore;
  float l_run = 0.f;            // this lane's share of the running sum
  f32x16 o[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) o[db] = f32x16{};

  // ---- epilogue of an item: O / l, lse = (m + log2 l) ln 2, then the state
  // is reset for the next item.  Lanes n and n + 32 hold the two halves of
  // row n, 4 consecutive d at a time.  bf16: one exchange between them gives
  // each lane 8 consecutive d, so each store is 16 bytes and a lane pair
  // writes 32 contiguous bytes of its row (half as many write requests as
  // 8-byte stores).
  auto epilogue = [&](const Item& e) __attribute__((always_inline)) {
    const int wt0 = e.tile * TW + tb * 32;
    const int qrow = wt0 + n;
    // lanes n and n + 32 share row n (and so this condition); the cross-lane
    // steps below run on all lanes, only the stores are conditional
    const bool row_ok = wt0 < e.Lq && qrow < e.Lq;
    const int h = e.hgrp * p.HW + hw;
    const float l_tot = sum_xor32(l_run);
    const float inv = 1.0f / l_tot;
    const int64_t orow = ((int64_t)(e.q0 + (row_ok ? qrow : 0)) * p.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      if constexpr (BF16) {
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          // x: this lane's 4 values of group 2 g2, y: of group 2 g2 + 1; the
          // swap of x's upper lanes with y's lower lanes leaves lane n (hh 0)
          // with d 8 (2 g2) + 0..7 and lane n + 32 with d 8 (2 g2 + 1) + 0..7
          const int r0 = 8 * g2, r1 = 8 * g2 + 4;
          const uint32_t x0 = pack_bf16x2(o[db][r0 + 0] * inv, o[db][r0 + 1] * inv);
          const uint32_t x1 = pack_bf16x2(o[db][r0 + 2] * inv, o[db][r0 + 3] * inv);
          const uint32_t y0 = pack_bf16x2(o[db][r1 + 0] * inv, o[db][r1 + 1] * inv);
          const uint32_t y1 = pack_bf16x2(o[db][r1 + 2] * inv, o[db][r1 + 3] * inv);
          const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
          const int d = db * 32 + (2 * g2 + hh) * 8;
          if (row_ok)
            *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) + orow + d) = u32x4{s0[0], s1[0], s0[1], s1[1]};
        }
      } else {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + g4 * 8 + hh * 4;
          if (row_ok)
            *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + orow + d) =
                f32x4{o[db][g4 * 4 + 0] * inv, o[db][g4 * 4 + 1] * inv, o[db][g4 * 4 + 2] * inv, o[db][g4 * 4 + 3] * inv};
        }
      }
    }
    if (p.lse && hh == 0 && row_ok) p.lse[(int64_t)(e.q0 + qrow) * p.Hq + h] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    m_run = kMaskedScore;
    l_run = 0.f;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) o[db] = f32x16{};
  };

  // ---- prologue: the first step -------------------------------------------
  Step cur;
  cur.it = item_from(0);
  cur.t = cur.it.t0;
  if (cur.it.ntiles == 0) return;   // no item for this workgroup (whole workgroup)
  Step nx1 = advance(cur);
  Step nx2 = advance(nx1);
  load_q(cur.it);
  int pg_nxt = load_pages(cur);
  issue_loads(pg_nxt, cur, 0);
  pg_nxt = load_pages(nx1);
  write_stage(0, cur);
  __syncthreads();

  for (int buf = 0;; buf ^= 1) {
    const Item& it = cur.it;
    const int t = cur.t;
    const bool has_next = nx1.it.ntiles != 0;
    const bool item_end = t + 1 == it.ntiles;   // last key tile of this item
    if (has_next) {
      issue_loads(pg_nxt, nx1, buf ^ 1);
      pg_nxt = load_pages(nx2);
    }

    const int kv0 = t * C::BN;
    const int cached = it.Lk - it.Lq;
    const int wt0 = it.tile * TW + tb * 32;
    const bool wave_live = wt0 < it.Lq;
    const int qpos = cached + wt0 + n;   // this lane's row's position among the keys
    bool skip = !wave_live || (p.causal && kv0 > cached + wt0 + 31);
    // a window: the tile lies wholly below every window of the wave's rows
    if constexpr (WIN) skip = skip || kv0 + C::BN <= cached + wt0 - p.window + 1;
    bool q_next = !(item_end && has_next);   // true once the next item's Q is on its way
    if (!skip) {
      bool need_mask = p.causal ? (kv0 + C::BN - 1 > cached + wt0) : (kv0 + C::BN > it.Lk);
      // ... or crosses the lower edge of some row's window
      if constexpr (WIN) need_mask = need_mask || kv0 < cached + wt0 + 32 - p.window;
      const char* Ks = smem + buf * C::STAGE;
      const char* Vs = Ks + C::KTILE;
      constexpr int NKB = C::BN / 32;
      f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
        const char* krow = Ks + (kb * 32 + n) * C::KROW;
        if constexpr (BF16) {
          // logical chunk 2 ks + hh of key kb*32 + n (whose swizzle is n's)
          const int kx = hh ^ C::kswz(n);
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks)
            s[kb] = mfma32x32x16_bf16(*reinterpret_cast<const u32x4*>(krow + ((2 * ks) ^ kx) * 16), qf[ks], s[kb]);
        } else {
#pragma unroll
          for (int c4 = 0; c4 < D / 8; ++c4) {
            const f32x4 a4 = *reinterpret_cast<const f32x4*>(krow + (hh * (D / 2) + c4 * 4) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) s[kb] = mfma32x32x2_f32(a4[e], qf[c4 * 4 + e], s[kb]);
          }
        }
      }
      // Q of this item is no longer needed: bring in the next item's
      if (!q_next) {
        load_q(nx1.it);
        q_next = true;
      }
      // Tile maximum.  Unmasked tiles take it over raw scores (c >= 0) and fold
      // the scale into the exponent's fma; tiles that cross the causal
      // diagonal, the key tail or a window's lower edge scale first and
      // select masked keys away.
      float mt = kMaskedScore;
      if (need_mask) {
        // key offset of register r inside a 32-key block: (r/4)*8 + hh*4 + r%4
        const int lim = (p.causal ? qpos + 1 : it.Lk) - kv0 - hh * 4;   // visible iff offset < lim
        const int lo = WIN ? qpos - p.window + 1 - kv0 - hh * 4 : 0;     // ... and offset >= lo
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = (r >> 2) * 8 + (r & 3) + kb * 32;
            const bool vis = off < lim && (!WIN || off >= lo);
            const float x = vis ? s[kb][r] * c : kMaskedScore;
            s[kb][r] = x;
            mt = fmaxf(mt, x);
          }
        }
        mt = max_xor32(mt);
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
        }
        mt = max_xor32(mt) * c;
      }
      if (__ballot(mt > m_run + kRescaleSlack)) {   // wave-uniform
        const float m_new = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) o[db] *= alpha;
      }
      float lsum = 0.f;
      if (need_mask) {
        // With a window a row may have seen no key yet (m_run still the mask
        // value): its masked scores are then taken against 0, so they give 0.
        const float m_ref = (WIN && m_run == kMaskedScore) ? 0.f : m_run;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(s[kb][r] - m_ref);
            s[kb][r] = e;
            lsum += e;
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -m_run));
            s[kb][r] = e;
            lsum += e;
          }
        }
      }
      l_run += lsum;
      // bf16: P rounded to bf16 (nearest even), the B operand of the PV MFMAs
      u32x4 pk[BF16 ? NKB : 1][2];
      if constexpr (BF16) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            pk[kb][pp] = u32x4{pack_bf16x2(s[kb][8 * pp + 0], s[kb][8 * pp + 1]),
                               pack_bf16x2(s[kb][8 * pp + 2], s[kb][8 * pp + 3]),
                               pack_bf16x2(s[kb][8 * pp + 4], s[kb][8 * pp + 5]),
                               pack_bf16x2(s[kb][8 * pp + 6], s[kb][8 * pp + 7])};
          }
        }
      }

      // O^T += V^T . P^T
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if constexpr (BF16) {
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            const u32x4 pb = pk[kb][pp];
            // k slot e of this MFMA is key kb*32 + 16 pp + 4 hh + (e % 4) + 8 (e / 4):
            // two transposing reads, keys +0..3 and +8..11 of the lane's group
            const char* vk = Vs + (kb * 32 + 16 * pp) * C::VROW + tr_row;
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) {
              const int cs = ((4 * db + tr_c) ^ tr_sw) * 16;
              const u32x2 lo2 = lds_read_tr16(vk + cs);
              const u32x2 hi2 = lds_read_tr16(vk + 8 * C::VROW + cs);
              o[db] = mfma32x32x16_bf16(u32x4{lo2[0], lo2[1], hi2[0], hi2[1]}, pb, o[db]);
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
            const float* vr = reinterpret_cast<const float*>(Vs + key * C::VROW);
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) o[db] = mfma32x32x2_f32(vr[db * 32 + n], s[kb][r], o[db]);
          }
        }
      }
    }
    if (!q_next) load_q(nx1.it);

    if (item_end) epilogue(it);

    if (has_next) write_stage(buf ^ 1, nx1);
    __syncthreads();
    if (!has_next) break;
    cur = nx1;
    nx1 = nx2;
    nx2 = advance(nx2);
  }
}

template <int D, bool BF16, int NW, bool WIN, bool KV8, bool I8 = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(AttnParams p) {
  prefill_body<D, BF16, NW, WIN, KV8, I8>(p, (int)gridDim.x, (int)blockIdx.x);
}

}  // namespace kvs
