// Decode attention (one query row per sequence) over the paged KV cache.
//
// Decode scans a long paged K/V context per sequence with few query rows, so it
// is bound by HBM bandwidth and needs its own load balancing (Transformer 추론
// 커널 (3/10), §13).  Long or uneven contexts are cut into pieces whose partial
// results (m_i, l_i, O_i) are merged afterwards in a numerically stable way
// (same page, §16), with the running-statistics update of §12.
//
// Work split.  The key blocks of the whole batch, laid end to end in sequence
// order (sequence b owns ceil(Lk_b / 16) of them; under a sliding window only
// those from the window's first block on), are cut into `nwg` equal
// contiguous ranges, one per workgroup, so every workgroup streams the same
// number of bytes whatever the length mix, and the grid is sized to be
// resident in one round (8 waves per CU on 256 CUs).  A range covers the tail
// of one sequence, whole sequences, and the head of another.  A workgroup walks
// its range as one continuous stream of steps (never crossing a sequence): the
// next step -- including the next sequence's query row -- is always being
// loaded while the current one is computed, so sequence switches cost no
// pipeline drain.  A sequence wholly inside the range is finished in place.
// A sequence cut by a range boundary leaves a normalised partial
// (O_i / l_i, lse_i) per piece.  The (at most two) pieces of a range are
// streamed first; each wave then adds their block counts to per-(sequence,
// KV head) counters, and the wave that completes a sequence merges its pieces
// in one round of loads:
//   lse = M + log2 sum 2^(lse_i - M),  out = sum 2^(lse_i - lse) O_i,
// then resets the counter, so no second launch is needed; the whole sequences
// of the range follow.  Partials and counts travel through device-scope
// stores, loads and atomics only (never agent-scope fences, which on this chip
// write back and invalidate a whole XCD's L2).
//
// Inside a workgroup, wave w handles KV head hg * hpw + w; the waves run
// independently (each has a private LDS slab).  Per wave:
//  * The G query heads that share the KV head ride in the 16 columns of the
//    MFMA (G <= 16; unused columns are zero), so each K/V byte is read once
//    for the whole group (§15).
//  * S^T = K . Q^T with the 16x16x32 bf16 MFMA: the A operand (16 keys x 32 d)
//    is one 16-byte global load per lane from the pool -- K goes straight from
//    HBM into registers.
//  * The accumulator layout of S^T (lane: one query column, 4 keys) is the B
//    operand layout of the 16x16x16 MFMA, so P feeds O^T = V^T . P^T directly.
//    V is transposed through the wave's LDS slab (d-major rows of 16 keys,
//    padded to 40 bytes so the 8-byte reads are bank-conflict free).
//  * All loads of a step are unconditional and masked at the point of use, so
//    the compiler can count outstanding loads exactly and a prefetch is never
//    waited on early.  Addresses past a sequence's end stay readable: tail
//    rows lie in an owned block, and blocks past a step's end read block 0.
#pragma once
#include <type_traits>

#include "kvs_device.hpp"
#include "kvs_internal.hpp"

namespace kvs {

// Phase timestamps (the KVS_PHASE_TIMES build, a profiling library of its
// own): thread 0 of each workgroup records the device's constant-rate clock
// (100 MHz) at the decode set-up and publish points into slot [workgroup][k]
// of a device array, read back by kvs_phase_times.  In the product build the
// probes are empty.
#ifdef KVS_PHASE_TIMES
constexpr int kPhaseSlots = 16;
static __device__ unsigned long long g_phase_t[4096][kPhaseSlots];
#define KVS_PHASE(k)                                                                              \
  do {                                                                                            \
    if (threadIdx.x == 0 && blockIdx.x < 4096) g_phase_t[blockIdx.x][k] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define KVS_PHASE(k) \
  do {               \
  } while (0)
#endif
// probe slots: 0 start, 7 lens and table staged (whole table), 1 block prefix,
// 10 table window, 2 new rows stored, 3 split pieces streamed, 5 partial
// stores complete, 6 merge counters, 8 the counters' completion bits, 4
// published and merged, 15 end
constexpr int kPhaseStart = 0, kPhaseStaged = 7, kPhasePrefix = 1, kPhaseWindow = 10, kPhaseNewRows = 2,
              kPhaseSplitDone = 3, kPhaseStores = 5, kPhaseCounters = 6, kPhaseFlags = 8, kPhaseMerged = 4,
              kPhaseEnd = 15;

template <int D, int NBS_ = 1>
struct DCfg {
  // 16-key blocks per step.  For bf16 / fp32 one block keeps the bytes in
  // flight near the bandwidth-latency product: a deeper prefetch only
  // lengthens the memory queues (and so the latency of every access,
  // including the publication of partials at the end), without raising the
  // throughput.  FP8 codes are half the bytes; kDecodeKv8Blocks sets their
  // blocks per step.
  static constexpr int NBS = NBS_;
  static constexpr int KI = D / 32;               // 16x16x32 k-steps over d
  static constexpr int NDB = D / 16;              // 16-wide d blocks of the output
  static constexpr int VROW = 40;                 // bytes per V^T row (16 keys + pad)
  static constexpr int VBLK = D * VROW;           // V^T bytes per 16-key block
  static constexpr int SLAB = NBS * VBLK;         // V^T bytes per wave (decode_slab_bytes)
  static constexpr int VIL = D / 64;              // (key pair, 8-d chunk) items per lane per block
  static constexpr int DPL = D / 64;              // d values per lane in the merge
};

constexpr int kTblWin = kDecodeTblWin;  // most blocks in one workgroup's range (its table entries sit in LDS)
// 16-byte table pieces a thread has in flight while staging the whole block
// table (a small batch's at most kDecodeSmallTbl entries: 8 per thread of an
// 8-wave workgroup)
constexpr int kStageLoads = 8;
// s_waitcnt immediate with vmcnt = 0 and the other counters left alone (gfx9
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;

// floor(x / d) for x < 2^52: a 32-bit division whenever x fits in 32 bits
// (the 64-bit division is a long instruction sequence).
__device__ __forceinline__ int64_t udiv_small(uint64_t x, uint32_t d) {
  if ((x >> 32) == 0) return (int64_t)((uint32_t)x / d);
  return (int64_t)(x / d);
}
// Sliding window W > 0: a sequence of L keys attends to keys L - W .. L - 1
// only, so only its blocks from (L - W) / 16 on enter the flattened axis.
__device__ __forceinline__ int first_block(int L, int W) { return W > 0 ? max(0, L - W) >> 4 : 0; }
__device__ __forceinline__ int seq_blocks(int L, int W) { return ((L + 15) >> 4) - first_block(L, W); }

// Start of range w on the flattened block axis: floor(w * total / nwg).
__device__ __forceinline__ int64_t range_start64(int64_t w, int total, int nwg) {
  return udiv_small((uint64_t)w * (uint32_t)total, (uint32_t)nwg);
}

// Cache-policy operand of the buffer intrinsics for device (agent) scope: the
// access goes to the device-wide coherence point, bypassing a stale or
// non-coherent copy in one XCD's L2.
constexpr int kDeviceScope = 16;
// Word 3 of a raw (untyped) buffer resource on gfx9.
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferWord3);
}

__device__ __forceinline__ float atomic_ld(const float* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_st(float* a, float v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One step of a workgroup's stream: up to NBS blocks of one sequence.
struct Step {
  int b;      // sequence (-1: no step; its loads are harmless dummies)
  int t;      // the sequence's query row
  int Lk;     // its key count
  int lblk;   // first block of the step, counted within the sequence
  int nblk;   // blocks in the step
  int gblk;   // first block of the step on the flattened axis
  int first;  // first step of this sequence's piece
  int last;   // last step of the piece
  int phys;   // RoPE step: physical block of the step (set with its loads)
};

// FP8 (E4M3) codes -> bf16, exactly (every E4M3 value is a bf16 value): the
// conversion instruction with unit scale, two codes per instruction.
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, bool hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 b2;
  const b2 r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                  : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  return *reinterpret_cast<const uint32_t*>(&r);
}
// 8 codes (d, d+1, .., d+7) -> 8 bf16 in the layout of a 16-byte bf16 chunk
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(const u32x2& w) {
  return u32x4{e4m3x2_to_bf16x2(w[0], false), e4m3x2_to_bf16x2(w[0], true), e4m3x2_to_bf16x2(w[1], false),
               e4m3x2_to_bf16x2(w[1], true)};
}
// 8 INT8 codes -> 8 bf16, exactly (an integer of magnitude <= 128 is a bf16
// value): each sign-extended byte converted to fp32, then packed
__device__ __forceinline__ u32x4 i8x8_to_bf16x8(const u32x2& w) {
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t u = w[h];
    r[2 * h] = pack_bf16x2((float)(int8_t)(u & 0xFFu), (float)(int8_t)((u >> 8) & 0xFFu));
    r[2 * h + 1] = pack_bf16x2((float)(int8_t)((u >> 16) & 0xFFu), (float)(int8_t)(u >> 24));
  }
  return r;
}
template <bool I8>
__device__ __forceinline__ u32x4 q8x8_to_bf16x8(const u32x2& w) {
  if constexpr (I8) return i8x8_to_bf16x8(w);
  else return e4m3x8_to_bf16x8(w);
}

// RoPE in the fused decode step: per wave, the cos / sin of the current
// sequence's angles in LDS, and this lane's frequency theta_lane.
template <bool ROPE>
struct DecodeRope {};
template <>
struct DecodeRope<true> {
  float* rcs = nullptr;   // [kRopeLdsPairs] cos, then [kRopeLdsPairs] sin
  double theta = 0.0;     // base^(-2 lane / rotary_dim) for lane < rotary_dim / 2
};
constexpr int kRopeLdsPairs = 64;
constexpr double kTwoPiHi = 6.283185307179586;       // 2 pi = hi + lo (hi the nearest double)
constexpr double kTwoPiLo = 2.4492935982947064e-16;

template <int D, bool BF16, bool APPEND, bool WIN, bool KV8, bool ROPE = false, bool I8 = false>
struct DecodeWave : DecodeRope<ROPE> {
  using C = DCfg<D, KV8 ? kDecodeKv8Blocks : 1>;
  static_assert(!ROPE || (BF16 && APPEND && !KV8), "RoPE: the bf16 fused decode step");
  static_assert(!I8 || KV8, "INT8 codes are a KV8 cache");
  using E = typename std::conditional<BF16, uint16_t, float>::type;
  // K / V elements: E4M3 codes when KV8 (then q and out are bf16)
  using KE = typename std::conditional<KV8, uint8_t, E>::type;
  // raw K / V registers of one 8-value chunk: 16 bytes of bf16 or 8 bytes of codes
  using KRaw = typename std::conditional<KV8, u32x2, u32x4>::type;
  static_assert(!KV8 || BF16, "FP8 caches: bf16 queries");
  static_assert(!(KV8 && APPEND) || C::NBS == 1, "FP8 fused step: one block per step");

  const AttnParams p;   // by value: a reference would pin the kernel arguments to scratch memory
  const int lane, col, grp, g;
  const bool head_ok;
  const int h;
  const int64_t tok_stride;
  const KE* kbase;
  const KE* vbase;
  char* slab;

  float m_run, l_run;
  f32x4 o[C::NDB];
  // the query fragments of the piece being computed (B operand of S^T =
  // K Q^T): loaded with a piece's first step only, kept across its steps
  u32x4 qc[C::KI];

  __device__ __forceinline__ DecodeWave(const AttnParams& p_, int g_, char* slab_)
      : p(p_), lane(threadIdx.x & 63), col(lane & 15), grp(lane >> 4), g(g_), head_ok(col < p_.G),
        h(g_ * p_.G + (col < p_.G ? col : 0)), tok_stride((int64_t)p_.Hkv * D),
        kbase(static_cast<const KE*>(p_.k) + (int64_t)g_ * D), vbase(static_cast<const KE*>(p_.v) + (int64_t)g_ * D),
        slab(slab_) {}

  __device__ __forceinline__ void reset() {
    m_run = kMaskedScore;
    l_run = 0.f;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) o[db] = f32x4{};
  }

  // s[j][r] holds the score of key k0 + 16 j + 4 grp + r for query column col;
  // on return it holds exp2(scaled score - running max).  Keys outside
  // [klo, kend) get a masked score by select (their K may be garbage).  Every
  // step holds at least one key of that range.
  template <int NB>
  __device__ __forceinline__ void softmax_update(f32x4 (&s)[NB], int k0, int kend, int klo) {
    float mt = kMaskedScore;
    const bool edge = k0 + 16 * NB > kend || (WIN && k0 < klo);
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = s[j][r] * p.scale_log2;
        const int key = k0 + 16 * j + grp * 4 + r;
        if (edge) x = (key < kend && (!WIN || key >= klo)) ? x : kMaskedScore;
        s[j][r] = x;
        mt = fmaxf(mt, x);
      }
    mt = max_xor32(max_xor16(mt));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __builtin_amdgcn_exp2f(s[j][r] - m_new);
        s[j][r] = e;
        lsum += e;
      }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) o[db] *= alpha;
  }

  // ---- bf16 path -----------------------------------------------------------
  struct NoScales {};
  struct Scales {
    f32x4 ks[C::NBS], vs[C::NBS];   // scales of the lane's 4 keys (4 grp .. 4 grp + 3)
  };
  // FP8 fused step: the new K / V rows (bf16), loaded with the step that holds
  // the new key; lane l holds elements D/64 l .. D/64 l + D/64 - 1 of each
  struct ScalesNew : Scales {
    uint32_t kn, vn;
  };
  using BufBase = typename std::conditional<KV8, typename std::conditional<APPEND, ScalesNew, Scales>::type,
                                            NoScales>::type;
  struct Buf : BufBase {
    KRaw k[C::NBS][C::KI];
    KRaw v[C::NBS][2 * C::VIL];
    u32x4 q[C::KI];   // the query row, loaded only with a piece's first step
  };
  // First element of sequence b's new K (V) row of this wave's KV head.
  __device__ __forceinline__ const E* new_row(const void* base, int b) const {
    return static_cast<const E*>(base) + ((int64_t)b * p.Hkv + g) * D;
  }

  // ---- append: the cache writes ---------------------------------------------
  // Workgroup w writes the new rows of sequences w, w + nwg, w + 2 nwg, ...
  // (its wave g the rows of KV head g) during its set-up, so the stores are
  // issued before its stream of loads starts.  One wave instruction covers RPI
  // rows: lane = row * CH + piece, one 16-byte piece per lane.  Rows whose
  // length or table entry lies outside the cache are skipped.
  static constexpr int EPP = 16 / (int)sizeof(E);   // elements per 16-byte piece
  static constexpr int CH = D / EPP;                // pieces per row of one KV head
  static constexpr int RPI = 64 / CH;               // rows per wave instruction
  struct NewRows {
    u32x4 k, v;
    int b;    // sequence of this lane's row (>= B: none)
    int kl;   // key index Lk - 1 (-1: no row for this lane)
    int pj;   // physical block holding it
  };
  // the rows of sequences b0 + stride * (lane / CH) (needs no lengths)
  __device__ __forceinline__ NewRows append_fetch(int b0, int stride) const {
    NewRows r;
    r.b = b0 + (lane / CH) * stride;
    r.kl = -1;
    r.pj = -1;
    if (r.b < p.B) {
      r.k = ld16(new_row(p.k_new, r.b) + (lane % CH) * EPP);
      r.v = ld16(new_row(p.v_new, r.b) + (lane % CH) * EPP);
    }
    return r;
  }
  // their slots: the length from LDS, the table entry from the staged whole
  // table (tbl_all) or else from memory
  __device__ __forceinline__ void append_locate(NewRows& r, const int* slens, const int* tbl_all) const {
    if (r.b < p.B) {
      const int Lk = slens[r.b];
      if (Lk >= 1 && Lk <= p.MB * kPage) {
        r.kl = Lk - 1;
        const int64_t at = (int64_t)r.b * p.MB + (r.kl >> 4);
        r.pj = tbl_all ? tbl_all[at] : p.table[at];
      }
    }
  }
  __device__ __forceinline__ NewRows append_load(int b0, int stride, const int* slens) const {
    NewRows r = append_fetch(b0, stride);
    append_locate(r, slens, nullptr);
    return r;
  }
  __device__ __forceinline__ void append_store(const NewRows& r) const {
    if (r.kl >= 0 && r.pj >= 0 && r.pj < p.NB) {
      const int64_t at = ((int64_t)r.pj * kPage + (r.kl & 15)) * tok_stride + (int64_t)g * D + (lane % CH) * EPP;
      st16(static_cast<E*>(p.k_cache_w) + at, r.k);
      st16(static_cast<E*>(p.v_cache_w) + at, r.v);
    }
  }
  // stores the rows `first` holds (those of sequences w + nwg * (lane / CH)),
  // then loads and stores the workgroup's remaining rows, if any
  __device__ __forceinline__ void append_rows(const NewRows& first, int w, int nwg, const int* slens) const {
    append_store(first);
    for (int b0 = w + nwg * RPI; b0 < p.B; b0 += nwg * RPI) append_store(append_load(b0, nwg, slens));
  }

  // K and V loads of one step.  With SUB, key kl is read from the new row
  // (kn, vn) instead of the cache (the cache slot is written in this launch).
  template <bool SUB>
  __device__ __forceinline__ void load_kv(const Step& st, const int* phys, Buf& bf, int kl, const E* kn,
                                          const E* vn) {
    const int kp = lane & 7;
#pragma unroll
    for (int j = 0; j < C::NBS; ++j) {
      const E* kblk = kbase + (int64_t)phys[j] * kPage * tok_stride;
      const E* vblk = vbase + (int64_t)phys[j] * kPage * tok_stride;
      const int key0 = (st.lblk + j) * 16;
#pragma unroll
      for (int i = 0; i < C::KI; ++i) {
        const E* ka = kblk + col * tok_stride + i * 32 + grp * 8;
        if constexpr (SUB) ka = key0 + col == kl ? kn + i * 32 + grp * 8 : ka;
        bf.k[j][i] = ld16_nt(ka);
      }
#pragma unroll
      for (int it = 0; it < C::VIL; ++it) {
        const int dch = (lane >> 3) + 8 * it;
        const E* va0 = vblk + (2 * kp) * tok_stride + dch * 8;
        const E* va1 = vblk + (2 * kp + 1) * tok_stride + dch * 8;
        if constexpr (SUB) {
          va0 = key0 + 2 * kp == kl ? vn + dch * 8 : va0;
          va1 = key0 + 2 * kp + 1 == kl ? vn + dch * 8 : va1;
        }
        bf.v[j][2 * it] = ld16_nt(va0);
        bf.v[j][2 * it + 1] = ld16_nt(va1);
      }
    }
  }

  // KV8: the codes of one step (8 bytes per 8-value chunk, the same lane
  // layout as the bf16 loads) and the scales of the lane's 4 keys.
  __device__ __forceinline__ void load_kv8(const int* phys, Buf& bf) {
    const int kp = lane & 7;
#pragma unroll
    for (int j = 0; j < C::NBS; ++j) {
      const KE* kblk = kbase + (int64_t)phys[j] * kPage * tok_stride;
      const KE* vblk = vbase + (int64_t)phys[j] * kPage * tok_stride;
#pragma unroll
      for (int i = 0; i < C::KI; ++i)
        bf.k[j][i] = ld8_nt(kblk + col * tok_stride + i * 32 + grp * 8);
#pragma unroll
      for (int it = 0; it < C::VIL; ++it) {
        const int dch = (lane >> 3) + 8 * it;
        bf.v[j][2 * it] = ld8_nt(vblk + (2 * kp) * tok_stride + dch * 8);
        bf.v[j][2 * it + 1] = ld8_nt(vblk + (2 * kp + 1) * tok_stride + dch * 8);
      }
      // scales [NB, Hkv, 16]: this head's 16 keys of the block are contiguous
      const int64_t so = ((int64_t)phys[j] * p.Hkv + g) * kPage + grp * 4;
      bf.ks[j] = ldf4_nt(p.k_scale + so);
      bf.vs[j] = ldf4_nt(p.v_scale + so);
    }
  }

  // Raw, unconditional loads of one step into `bf` (phys[j] = physical block of
  // the step's j-th block, 0 for blocks past its end).
  __device__ __forceinline__ void load(const Step& st, const int* phys, Buf& bf) {
    // the query row comes with the first step of a piece (a wave-uniform
    // branch); later steps of the piece reuse it
    if (st.first) {
      const int hq = st.b < 0 ? 0 : h;
      const E* qp = static_cast<const E*>(p.q) + ((int64_t)(st.b < 0 ? 0 : st.t) * p.Hq + hq) * D;
#pragma unroll
      for (int i = 0; i < C::KI; ++i) bf.q[i] = ld16(qp + i * 32 + grp * 8);
    }
    if constexpr (KV8) {
      load_kv8(phys, bf);
      if constexpr (APPEND) {
        // the step holding key Lk - 1 also brings in the new rows
        const int kl = st.Lk - 1;
        if (st.b >= 0 && (kl >> 4) == st.lblk) {   // wave-uniform
          const E* kn = new_row(p.k_new, st.b);
          const E* vn = new_row(p.v_new, st.b);
          if constexpr (D == 64) {
            bf.kn = kn[lane];
            bf.vn = vn[lane];
          } else {
            bf.kn = *reinterpret_cast<const uint32_t*>(kn + 2 * lane);
            bf.vn = *reinterpret_cast<const uint32_t*>(vn + 2 * lane);
          }
        }
      }
    } else if constexpr (APPEND) {
      // append: the step holding key kl = Lk - 1 (one step per sequence, a
      // wave-uniform branch) reads that key from the new row; the cache slot
      // is written elsewhere in the same launch
      const int kl = st.Lk - 1;
      const bool app = st.b >= 0 && (kl >> 4) >= st.lblk && (kl >> 4) < st.lblk + C::NBS;
      if (app) {
        load_kv<true>(st, phys, bf, kl, new_row(p.k_new, st.b), new_row(p.v_new, st.b));
      } else {
        load_kv<false>(st, phys, bf, 0, nullptr, nullptr);
      }
    } else {
      load_kv<false>(st, phys, bf, 0, nullptr, nullptr);
    }
  }

  // ---- RoPE (fused decode step) ---------------------------------------------
  // The angles of the new token of a sequence of Lk keys (position Lk - 1):
  // lane i < rotary_dim / 2 forms pair i's angle in double (the product and
  // its reduction by 2 pi), then cos / sin in fp32, into this wave's LDS.
  __device__ __forceinline__ void rope_angles(int Lk) {
    if constexpr (ROPE) {
      if (lane < (p.rope_rd >> 1)) {
        const double a = (double)(Lk - 1) * p.rope_inv_scale * this->theta;
        const double k = rint(a * (1.0 / kTwoPiHi));
        const double r = fma(-k, kTwoPiHi, a) - k * kTwoPiLo;
        float sn, cs;
        sincosf((float)r, &sn, &cs);
        this->rcs[lane] = cs;
        this->rcs[kRopeLdsPairs + lane] = sn;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    }
  }
  // Rotates this lane's chunks x[i] (value e of chunk i is d = 32 i + 8 grp + e,
  // the lane layout of both the query and a key row): neox pairs (d, d + rd/2)
  // are chunks i and i + rd/64 of the same lane, interleaved pairs are
  // neighbours inside a chunk.  Results are rounded to bf16.
  __device__ __forceinline__ void rope_rotate(u32x4 (&x)[C::KI]) const {
    if constexpr (ROPE) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (p.rope_style == 0) {
        const int ni = p.rope_rd >> 6;
#pragma unroll
        for (int i = 0; i < C::KI / 2 + (C::KI == 1 ? 1 : 0); ++i) {
          if (i >= ni || i + ni >= C::KI) continue;
          const int j0 = 32 * i + 8 * grp;
          const f32x4 c0 = *reinterpret_cast<const f32x4*>(this->rcs + j0);
          const f32x4 c1 = *reinterpret_cast<const f32x4*>(this->rcs + j0 + 4);
          const f32x4 s0 = *reinterpret_cast<const f32x4*>(this->rcs + kRopeLdsPairs + j0);
          const f32x4 s1 = *reinterpret_cast<const f32x4*>(this->rcs + kRopeLdsPairs + j0 + 4);
          u32x4& a = x[i];
          u32x4& b = x[i + ni];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float cl = w < 2 ? c0[2 * w] : c1[2 * w - 4], ch = w < 2 ? c0[2 * w + 1] : c1[2 * w - 3];
            const float sl = w < 2 ? s0[2 * w] : s1[2 * w - 4], sh = w < 2 ? s0[2 * w + 1] : s1[2 * w - 3];
            const float a0 = bf16lo_to_f32(a[w]), a1 = bf16hi_to_f32(a[w]);
            const float b0 = bf16lo_to_f32(b[w]), b1 = bf16hi_to_f32(b[w]);
            a[w] = pack_bf16x2(fmaf(a0, cl, -b0 * sl), fmaf(a1, ch, -b1 * sh));
            b[w] = pack_bf16x2(fmaf(b0, cl, a0 * sl), fmaf(b1, ch, a1 * sh));
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < C::KI; ++i) {
          if (32 * i + 8 * grp >= p.rope_rd) continue;
          const int j0 = 16 * i + 4 * grp;
          const f32x4 c = *reinterpret_cast<const f32x4*>(this->rcs + j0);
          const f32x4 sn = *reinterpret_cast<const f32x4*>(this->rcs + kRopeLdsPairs + j0);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float x1 = bf16lo_to_f32(x[i][w]), x2 = bf16hi_to_f32(x[i][w]);
            x[i][w] = pack_bf16x2(fmaf(x1, c[w], -x2 * sn[w]), fmaf(x2, c[w], x1 * sn[w]));
          }
        }
      }
    }
  }
  // the cache slot (element offset of this wave's head) of key kl of block phys
  __device__ __forceinline__ int64_t slot_offset(int phys, int kl) const {
    return ((int64_t)phys * kPage + (kl & 15)) * tok_stride + (int64_t)g * D;
  }

  // first key of sequence st.b that the query row sees (the window's start)
  __device__ __forceinline__ int first_key(const Step& st) const { return WIN ? max(0, st.Lk - p.window) : 0; }

  // FP8 fused step: quantize the new K and V rows exactly as kv_store_paged_fp8
  // does (absmax of the row over the lanes holding it, s = absmax / 448, codes
  // of x / s), put codes and scales in place of the unwritten slot's, and write
  // them to the cache.  K row: lanes col == r (4 lanes, grp 0..3); V row: the 8
  // lanes with 2 kp (or 2 kp + 1) == r; r = kl - k0.
  __device__ __forceinline__ void new_rows_fp8(const Step& st, Buf& b) const {
    if constexpr (KV8 && APPEND) {
      const int kl = st.Lk - 1, k0 = st.lblk * 16;
      if (kl < k0 || kl >= k0 + 16) return;   // wave-uniform
      const int r = kl - k0, kp = lane & 7;
      // The row's absmax over the wave, the scale and codes as in
      // kv_store_paged_fp8 (same fp32 divisions, same code function), each
      // lane coding its own D/64 elements of each row.
      constexpr int EPL = D / 64;
      static_assert(EPL == 1 || EPL == 2, "D is 64 or 128");
      float xk[EPL], xv[EPL];
      xk[0] = bf16lo_to_f32(b.kn);
      xv[0] = bf16lo_to_f32(b.vn);
      if constexpr (EPL == 2) {
        xk[1] = bf16hi_to_f32(b.kn);
        xv[1] = bf16hi_to_f32(b.vn);
      }
      float ak = fabsf(xk[0]), av = fabsf(xv[0]);
      if constexpr (EPL == 2) {
        ak = fmaxf(ak, fabsf(xk[1]));
        av = fmaxf(av, fabsf(xv[1]));
      }
      constexpr float QMAX = I8 ? 127.f : 448.f;
      const float sk = wave_max(ak) / QMAX;   // the same in every lane
      const float sv = wave_max(av) / QMAX;
      uint32_t ck = 0u, cv = 0u;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        if (sk > 0.f) ck |= (I8 ? i8_code(xk[e] / sk) : e4m3_code(xk[e] / sk)) << (8 * e);
        if (sv > 0.f) cv |= (I8 ? i8_code(xv[e] / sv) : e4m3_code(xv[e] / sv)) << (8 * e);
      }
      // The codes go through the first 2 D bytes of this wave's slab (which
      // the step's V^T overwrites afterwards) to the lanes that hold key r:
      // K chunks i 32 + grp 8 (lanes col == r), V chunks dch (lanes of key
      // pair kp holding r).  One wave's LDS operations execute in order.
      uint8_t* cb = reinterpret_cast<uint8_t*>(slab);
      if constexpr (EPL == 1) {
        cb[lane] = (uint8_t)ck;
        cb[D + lane] = (uint8_t)cv;
      } else {
        *reinterpret_cast<uint16_t*>(cb + 2 * lane) = (uint16_t)ck;
        *reinterpret_cast<uint16_t*>(cb + D + 2 * lane) = (uint16_t)cv;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      if (col == r) {
#pragma unroll
        for (int i = 0; i < C::KI; ++i) b.k[0][i] = *reinterpret_cast<const u32x2*>(cb + i * 32 + grp * 8);
      }
#pragma unroll
      for (int it = 0; it < C::VIL; ++it) {
        const u32x2 vc = *reinterpret_cast<const u32x2*>(cb + D + ((lane >> 3) + 8 * it) * 8);
        if (2 * kp == r) b.v[0][2 * it] = vc;
        if (2 * kp + 1 == r) b.v[0][2 * it + 1] = vc;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      const float skr = sk, svr = sv;
      const bool store = st.phys >= 0 && st.phys < p.NB;
      const int64_t so = slot_offset(st.phys, kl);
      if (store) {
        uint8_t* kd = static_cast<uint8_t*>(p.k_cache_w) + so;
        uint8_t* vd = static_cast<uint8_t*>(p.v_cache_w) + so;
        if constexpr (EPL == 1) {
          kd[lane] = (uint8_t)ck;
          vd[lane] = (uint8_t)cv;
        } else {
          *reinterpret_cast<uint16_t*>(kd + 2 * lane) = (uint16_t)ck;
          *reinterpret_cast<uint16_t*>(vd + 2 * lane) = (uint16_t)cv;
        }
      }
      // the lanes holding key r's scales (keys 4 grp .. 4 grp + 3)
      if (grp == (r >> 2)) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          b.ks[0][q4] = q4 == (r & 3) ? skr : b.ks[0][q4];
          b.vs[0][q4] = q4 == (r & 3) ? svr : b.vs[0][q4];
        }
      }
      if (store && lane == 0) {
        const int64_t si = ((int64_t)st.phys * p.Hkv + g) * kPage + (kl & 15);
        p.k_scale_w[si] = skr;
        p.v_scale_w[si] = svr;
      }
    }
  }

  __device__ __forceinline__ void compute(const Step& st, const Buf& bf) {
    // FP8 fused step: the new rows' codes go into the step's own buffer (one
    // of the stream's two, reloaded after this step)
    if constexpr (KV8 && APPEND) new_rows_fp8(st, const_cast<Buf&>(bf));
    const int k0 = st.lblk * 16;
    const int kend = min(st.Lk, (st.lblk + st.nblk) * 16);
    const int klo = first_key(st);
    const bool edge = k0 + 16 * C::NBS > kend || (WIN && k0 < klo);
    const u32x4 zero = {0, 0, 0, 0};
    // V^T into the slab: word (V[2kp][d], V[2kp+1][d]) at row d, key pair kp.
    // The slab is private to this wave and LDS operations of one wave execute
    // in order, so a compiler-level fence is all the ordering needed.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int j = 0; j < C::NBS; ++j) {
      const int kp = lane & 7;
      const int kv = k0 + 16 * j + 2 * kp;
      const bool v0_ok = !edge || (kv < kend && (!WIN || kv >= klo));
      const bool v1_ok = !edge || (kv + 1 < kend && (!WIN || kv + 1 >= klo));
#pragma unroll
      for (int it = 0; it < C::VIL; ++it) {
        const int dch = (lane >> 3) + 8 * it;
        u32x4 w0, w1;
        if constexpr (KV8) {
          w0 = v0_ok ? q8x8_to_bf16x8<I8>(bf.v[j][2 * it]) : zero;
          w1 = v1_ok ? q8x8_to_bf16x8<I8>(bf.v[j][2 * it + 1]) : zero;
        } else {
          w0 = v0_ok ? bf.v[j][2 * it] : zero;
          w1 = v1_ok ? bf.v[j][2 * it + 1] : zero;
        }
        if constexpr (ROPE) {
          // the new token's V row (read from v_new) goes to its cache slot
          const int kl = st.Lk - 1;
          if (st.phys >= 0 && st.phys < p.NB) {
            if (kv == kl) st16(static_cast<E*>(p.v_cache_w) + slot_offset(st.phys, kl) + dch * 8, bf.v[j][2 * it]);
            if (kv + 1 == kl) st16(static_cast<E*>(p.v_cache_w) + slot_offset(st.phys, kl) + dch * 8, bf.v[j][2 * it + 1]);
          }
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          char* r0 = slab + j * C::VBLK + (dch * 8 + 2 * m) * C::VROW + kp * 4;
          *reinterpret_cast<uint32_t*>(r0) = __builtin_amdgcn_perm(w1[m], w0[m], 0x05040100u);
          *reinterpret_cast<uint32_t*>(r0 + C::VROW) = __builtin_amdgcn_perm(w1[m], w0[m], 0x07060302u);
        }
      }
    }
    if (st.first) {
#pragma unroll
      for (int i = 0; i < C::KI; ++i) qc[i] = head_ok ? bf.q[i] : zero;
      if constexpr (ROPE) rope_rotate(qc);
    }
    const u32x4 (&q)[C::KI] = qc;
    f32x4 s[C::NBS];
#pragma unroll
    for (int j = 0; j < C::NBS; ++j) {
      s[j] = f32x4{};
      if constexpr (ROPE) {
        // the step holding the new key kl = Lk - 1 (read from k_new): rotate
        // that key row (lanes col == kl - k0) and write it to its cache slot
        u32x4 kk[C::KI];
#pragma unroll
        for (int i = 0; i < C::KI; ++i) kk[i] = bf.k[j][i];
        const int kl = st.Lk - 1;
        if (kl >= k0 + 16 * j && kl < k0 + 16 * j + 16) {   // wave-uniform
          u32x4 kr[C::KI];
#pragma unroll
          for (int i = 0; i < C::KI; ++i) kr[i] = kk[i];
          rope_rotate(kr);
          if (col == kl - k0 - 16 * j) {
#pragma unroll
            for (int i = 0; i < C::KI; ++i) kk[i] = kr[i];
            if (st.phys >= 0 && st.phys < p.NB) {
#pragma unroll
              for (int i = 0; i < C::KI; ++i)
                st16(static_cast<E*>(p.k_cache_w) + slot_offset(st.phys, kl) + i * 32 + grp * 8, kk[i]);
            }
          }
        }
#pragma unroll
        for (int i = 0; i < C::KI; ++i) s[j] = mfma16x16x32_bf16(kk[i], q[i], s[j]);
      } else {
#pragma unroll
        for (int i = 0; i < C::KI; ++i) {
          if constexpr (KV8) s[j] = mfma16x16x32_bf16(q8x8_to_bf16x8<I8>(bf.k[j][i]), q[i], s[j]);
          else s[j] = mfma16x16x32_bf16(bf.k[j][i], q[i], s[j]);
        }
      }
      // KV8: K = code * scale of its key, so the score is scaled per key
      if constexpr (KV8) {
#pragma unroll
        for (int r = 0; r < 4; ++r) s[j][r] *= bf.ks[j][r];
      }
    }
    softmax_update<C::NBS>(s, k0, kend, klo);
    if constexpr (KV8) {
      // V = code * scale of its key: P carries the scale into the PV product
      // (after l has summed the unscaled P).  Keys outside the range get 0,
      // not 0 * an unwritten scale.
#pragma unroll
      for (int j = 0; j < C::NBS; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + 16 * j + grp * 4 + r;
          const bool ok = !edge || (key < kend && (!WIN || key >= klo));
          s[j][r] = ok ? s[j][r] * bf.vs[j][r] : 0.f;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int j = 0; j < C::NBS; ++j) {
      const u32x2 pb = {pack_bf16x2(s[j][0], s[j][1]), pack_bf16x2(s[j][2], s[j][3])};
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const u32x2 a = *reinterpret_cast<const u32x2*>(slab + j * C::VBLK + (db * 16 + col) * C::VROW + grp * 8);
        o[db] = mfma16x16x16_bf16(a, pb, o[db]);
      }
    }
  }

  // ---- fp32 path: 16x16x4 MFMA, one element per lane per operand ------------
  // k-slot grp of k-step i covers d = grp * D/4 + i.  Not pipelined.
  __device__ __forceinline__ void compute_f32(const Step& st, const int* phys) {
    constexpr int QF = D / 4;
    const float* qp = static_cast<const float*>(p.q) + ((int64_t)st.t * p.Hq + h) * D;
    float qv[QF];
#pragma unroll
    for (int c4 = 0; c4 < QF / 4; ++c4) {
      const u32x4 w = ld16_keep(qp + grp * QF + c4 * 4, head_ok);
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[c4 * 4 + e] = __uint_as_float(w[e]);
    }
    const float* kb = reinterpret_cast<const float*>(kbase);
    const float* vb = reinterpret_cast<const float*>(vbase);
    const int kend = min(st.Lk, (st.lblk + st.nblk) * 16);
    const int klo = first_key(st);
    // append: key kl = Lk - 1 comes from the new row
    const int kl = st.Lk - 1;
    const float* kn = nullptr;
    const float* vn = nullptr;
    bool app = false;
    if constexpr (APPEND) {
      app = (kl >> 4) >= st.lblk && (kl >> 4) < st.lblk + st.nblk;   // uniform
      kn = reinterpret_cast<const float*>(new_row(p.k_new, st.b));
      vn = reinterpret_cast<const float*>(new_row(p.v_new, st.b));
    }
#pragma unroll
    for (int j = 0; j < C::NBS; ++j) {
      if (j >= st.nblk) break;
      const int kb0 = (st.lblk + j) * 16;
      const float* kblk = kb + (int64_t)phys[j] * kPage * tok_stride;
      const float* vblk = vb + (int64_t)phys[j] * kPage * tok_stride;
      f32x4 s[1] = {f32x4{}};
#pragma unroll
      for (int c4 = 0; c4 < QF / 4; ++c4) {
        const float* ka = kblk + col * tok_stride + grp * QF + c4 * 4;
        if constexpr (APPEND) ka = (app && kb0 + col == kl) ? kn + grp * QF + c4 * 4 : ka;
        const u32x4 w = ld16(ka);
#pragma unroll
        for (int e = 0; e < 4; ++e) s[0] = mfma16x16x4_f32(__uint_as_float(w[e]), qv[c4 * 4 + e], s[0]);
      }
      softmax_update<1>(s, kb0, kend, klo);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = grp * 4 + r;
        const bool ok = kb0 + key < kend && (!WIN || kb0 + key >= klo);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          float v = vblk[key * tok_stride + db * 16 + col];
          if constexpr (APPEND) v = (app && kb0 + key == kl) ? vn[db * 16 + col] : v;
          o[db] = mfma16x16x4_f32(ok ? v : 0.f, s[0][r], o[db]);
        }
      }
    }
  }

  // ---- end of a piece ------------------------------------------------------
  // Combine the 4 lane groups' shares of l; returns the base-2 lse.
  __device__ __forceinline__ float finish(float* inv_out) {
    const float l_tot = sum_xor32(sum_xor16(l_run));
    *inv_out = 1.0f / l_tot;
    return m_run + __builtin_amdgcn_logf(l_tot);
  }

  __device__ __forceinline__ void store_final(int t) {
    float inv;
    const float lse2 = finish(&inv);
    if (!head_ok) return;
    const int64_t orow = ((int64_t)t * p.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int d = db * 16 + grp * 4;
      const float a0 = o[db][0] * inv, a1 = o[db][1] * inv, a2 = o[db][2] * inv, a3 = o[db][3] * inv;
      if constexpr (BF16) {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + orow + d) =
            u32x2{pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + orow + d) = f32x4{a0, a1, a2, a3};
      }
    }
    if (p.lse && grp == 0) p.lse[(int64_t)t * p.Hq + h] = lse2 * kLn2;
  }

  // Bytes of the partial-output array [nwg + B, Hq, D] (the planner keeps it
  // below 2 GiB, so 32-bit buffer offsets reach all of it).
  __device__ __forceinline__ uint32_t part_bytes() const {
    return (uint32_t)(p.nwg + p.B) * (uint32_t)p.Hq * (uint32_t)(D * 4);
  }

  // Partials are published with device-scope stores (written through to the
  // device-wide coherence point); nothing waits for them here.
  __device__ __forceinline__ void store_partial(int slot) {
    float inv;
    const float lse2 = finish(&inv);
    if (!head_ok) return;
    const uint32_t prow = (uint32_t)slot * (uint32_t)p.Hq + (uint32_t)h;
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(p.part_o, part_bytes());
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const u32x4 v = {__float_as_uint(o[db][0] * inv), __float_as_uint(o[db][1] * inv),
                       __float_as_uint(o[db][2] * inv), __float_as_uint(o[db][3] * inv)};
      __builtin_amdgcn_raw_buffer_store_b128(v, rs, (prow * D + db * 16 + grp * 4) * 4, 0, kDeviceScope);
    }
    if (grp == 0) atomic_st(p.part_lse + prow, lse2);
  }

  // A split piece that finishes while the range's other split piece is still
  // to be streamed is held in registers and stored with that one: a store in
  // the middle of the stream would hold up the loads after it (they retire
  // in order with it), for a full write round trip.
  f32x4 ho[C::NDB];
  float hlse;
  uint32_t hslot;
  __device__ __forceinline__ void hold_partial(int slot) {
    float inv;
    hlse = finish(&inv);
    hslot = (uint32_t)slot;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) ho[db] = f32x4{o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv};
  }
  __device__ __forceinline__ void store_held() {
    if (!head_ok) return;
    const uint32_t prow = hslot * (uint32_t)p.Hq + (uint32_t)h;
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(p.part_o, part_bytes());
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const u32x4 v = {__float_as_uint(ho[db][0]), __float_as_uint(ho[db][1]), __float_as_uint(ho[db][2]),
                       __float_as_uint(ho[db][3])};
      __builtin_amdgcn_raw_buffer_store_b128(v, rs, (prow * D + db * 16 + grp * 4) * 4, 0, kDeviceScope);
    }
    if (grp == 0) atomic_st(p.part_lse + prow, hlse);
  }

  // ---- merge of split sequences ---------------------------------------------
  // The pieces of sequence b (query row b, blocks [sb0, sb1) on the flattened
  // axis) are the partial slots w + b of the workgroups w whose ranges meet
  // its blocks.  A merging wave works through units -- HB heads by PC pieces,
  // the pieces counted from the sequence's first -- and loads the next unit
  // while it combines the current one.  In a unit, lane i loads the lse of
  // (piece i / HB, head j = i % HB) and every lane loads its d = lane + 64 k of
  // each (piece, head) output.  The lanes of head j then hold that head's
  // running maximum M and weight sum W (cross-lane reductions), and each
  // output element adds the unit's pieces with independent fmas:
  //   M' = max(M, max_i lse_i),  W' = W 2^(M - M') + sum_i 2^(lse_i - M'),
  //   acc' = acc 2^(M - M') + sum_i 2^(lse_i - M') O_i,   out = acc / W.
  // A sequence's arithmetic is the same whichever workgroup merges it and
  // whatever else that wave merges, so repeated calls give the same bits.
  static constexpr int HB = 4;
  static constexpr int PC = 8;
  struct MUnit {
    int b;     // sequence (< 0: no unit)
    int t;     // its query row (the row of out and lse)
    int wf;    // range holding its first block
    int npc;   // its pieces
    int qh0;   // first head of the unit (within the wave's G)
    int i0;    // first piece of the unit
  };
  struct MBuf {
    float ov[PC][HB][C::DPL];
    float lsl;        // this lane's lse (piece i / HB, head i % HB), or masked
    uint64_t live;    // live pieces of the unit
  };
  __device__ __forceinline__ MUnit merge_first(int b, int t, int sb0, int sb1, int total, int nwg) const {
    MUnit u;
    u.b = b;
    u.t = t;
    // ranges holding the first and the last block of the sequence
    u.wf = (int)udiv_small((uint64_t)(sb0 + 1) * (uint32_t)nwg - 1, (uint32_t)total);
    const int wl = (int)udiv_small((uint64_t)sb1 * (uint32_t)nwg - 1, (uint32_t)total);
    u.npc = wl - u.wf + 1;
    u.qh0 = 0;
    u.i0 = 0;
    return u;
  }
  __device__ __forceinline__ void merge_load(const MUnit& u, MBuf& mb, int total, int nwg,
                                             __amdgpu_buffer_rsrc_t rs) const {
    if (u.b < 0) return;
    // piece i of the unit -> its range; pieces past the sequence's last reuse
    // that one's slot (a readable address) and are not live
    const int nround = min(PC, u.npc - u.i0);
    auto range = [&](int i) __attribute__((always_inline)) { return u.wf + u.i0 + min(i, nround - 1); };
    // with at least as many blocks as ranges every range is non-empty,
    // otherwise lane i checks piece i
    if (total >= nwg) {
      mb.live = nround >= 64 ? ~0ull : ((1ull << nround) - 1);
    } else {
      const int wr = range(lane);
      mb.live = __ballot(lane < nround && range_start64(wr + 1, total, nwg) > range_start64(wr, total, nwg));
    }
    {
      const int il = (lane % (PC * HB)) / HB;
      const int hh = g * p.G + min(u.qh0 + lane % HB, p.G - 1);
      const float l = atomic_ld(p.part_lse + (int64_t)(range(il) + u.b) * p.Hq + hh);
      mb.lsl = (lane < PC * HB && ((mb.live >> il) & 1)) ? l : kMaskedScore;
    }
#pragma unroll
    for (int i = 0; i < PC; ++i) {
      const uint32_t slot = (uint32_t)(range(i) + u.b);
#pragma unroll
      for (int j = 0; j < HB; ++j) {
        const uint32_t hh = (uint32_t)(g * p.G + min(u.qh0 + j, p.G - 1));
#pragma unroll
        for (int k = 0; k < C::DPL; ++k)
          mb.ov[i][j][k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              rs, ((slot * (uint32_t)p.Hq + hh) * D + lane + 64 * k) * 4, 0, kDeviceScope));
      }
    }
  }
  __device__ __forceinline__ void merge_combine(const MBuf& mb, float& M, float& W, float (&acc)[HB][C::DPL]) const {
    static_assert(HB == 4, "the reductions below run over the lanes that share lane % 4");
    const float Mn = fmaxf(M, max_mod4(mb.lsl));
    const float sc = __builtin_amdgcn_exp2f(M - Mn);
    const float wt = mb.lsl == kMaskedScore ? 0.f : __builtin_amdgcn_exp2f(mb.lsl - Mn);
    W = W * sc + sum_mod4(wt);
    M = Mn;
#pragma unroll
    for (int j = 0; j < HB; ++j) {
      const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), j));
#pragma unroll
      for (int k = 0; k < C::DPL; ++k) acc[j][k] *= f;
    }
#pragma unroll
    for (int i = 0; i < PC; ++i) {
      // uniform: pieces that do not exist are skipped, never weighted by 0
      if (!((mb.live >> i) & 1)) continue;
#pragma unroll
      for (int j = 0; j < HB; ++j) {
        const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), i * HB + j));
#pragma unroll
        for (int k = 0; k < C::DPL; ++k) acc[j][k] = fmaf(f, mb.ov[i][j][k], acc[j][k]);
      }
    }
  }
  __device__ __forceinline__ void merge_store(const MUnit& u, float M, float W, const float (&acc)[HB][C::DPL]) const {
#pragma unroll
    for (int j = 0; j < HB; ++j) {
      if (u.qh0 + j >= p.G) break;
      const int hh = g * p.G + u.qh0 + j;
      const float Wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(W), j));
      const float Mj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(M), j));
      const float inv = 1.0f / Wj;
      const int64_t orow = ((int64_t)u.t * p.Hq + hh) * D;
#pragma unroll
      for (int k = 0; k < C::DPL; ++k) {
        if constexpr (BF16) {
          reinterpret_cast<__bf16*>(p.out)[orow + lane + 64 * k] = (__bf16)(acc[j][k] * inv);
        } else {
          static_cast<float*>(p.out)[orow + lane + 64 * k] = acc[j][k] * inv;
        }
      }
      if (p.lse && lane == 0) p.lse[(int64_t)u.t * p.Hq + hh] = (Mj + __builtin_amdgcn_logf(Wj)) * kLn2;
    }
  }
  // Merges sequence b0 (query row t0, blocks [s00, s10)) and, if nm == 2,
  // sequence b1 (row t1, blocks [s01, s11)), the units of both in one
  // pipelined pass.
  __device__ __forceinline__ void merge(int nm, int b0, int t0, int s00, int s10, int b1, int t1, int s01, int s11,
                                        int total, int nwg) {
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(p.part_o, part_bytes());
    auto next = [&](const MUnit& u) __attribute__((always_inline)) {
      MUnit n = u;
      n.i0 += PC;
      if (n.i0 >= u.npc) {
        n.i0 = 0;
        n.qh0 += HB;
        if (n.qh0 >= p.G) {
          if (nm == 2 && u.b == b0) {
            n = merge_first(b1, t1, s01, s11, total, nwg);
          } else {
            n.b = -1;
          }
        }
      }
      return n;
    };
    float M = kMaskedScore, W = 0.f;
    float acc[HB][C::DPL];
    auto step = [&](const MUnit& cur, const MBuf& mb) __attribute__((always_inline)) {
      if (cur.i0 == 0) {
        M = kMaskedScore;
        W = 0.f;
#pragma unroll
        for (int j = 0; j < HB; ++j)
#pragma unroll
          for (int k = 0; k < C::DPL; ++k) acc[j][k] = 0.f;
      }
      merge_combine(mb, M, W, acc);
      if (cur.i0 + PC >= cur.npc) merge_store(cur, M, W, acc);
    };
    MBuf bA, bB;
    MUnit cur = merge_first(b0, t0, s00, s10, total, nwg);
    merge_load(cur, bA, total, nwg, rs);
    for (;;) {
      MUnit nxt = next(cur);
      merge_load(nxt, bB, total, nwg, rs);
      step(cur, bA);
      if (nxt.b < 0) break;
      cur = nxt;
      nxt = next(cur);
      merge_load(nxt, bA, total, nwg, rs);
      step(cur, bB);
      if (nxt.b < 0) break;
      cur = nxt;
    }
  }
};

// One workgroup's part of decode: range w of nwg along the flattened block
// axis, KV heads hg * hpw .. hg * hpw + hpw - 1.  I8: the KV8 caches hold INT8
// codes, not E4M3.  MIX: the decode part of a mixed launch -- the flattened
// axis holds only the sequences with one query row (in batch order), each
// answered at its own query row cu_seqlens_q[b].
template <int D, bool BF16, bool APPEND, bool WIN, bool KV8, bool ROPE, bool I8 = false, bool MIX = false>
__device__ __forceinline__ void decode_body(AttnParams p, const int w, const int hg, const int nwg) {
  static_assert(!MIX || (!APPEND && !ROPE && !KV8), "a mixed launch's decode part is plain attention");
  using C = DCfg<D, KV8 ? kDecodeKv8Blocks : 1>;
  using W = DecodeWave<D, BF16, APPEND, WIN, KV8, ROPE, I8>;
  // RoPE: the new rows are written by the waves that attend them (rotated),
  // not during set-up
  constexpr bool SETUP_APPEND = APPEND && !ROPE && !KV8;
  constexpr int RB = ROPE ? 2 * kRopeLdsPairs * (int)sizeof(float) : 0;   // per-wave cos / sin
  const int win = WIN ? p.window : 0;   // sliding window (0: none)
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int B = p.B;
  int* slens = reinterpret_cast<int*>(smem);         // [B]      seqlens_k
  int* sstart = slens + ((B + 3) & ~3);              // [B + 1]  exclusive block prefix
  // MIX: sequence i of the flattened axis is batch sequence sseq[i], its
  // query row srow[i]
  int* sseq = sstart + ((B + 1 + 3) & ~3);
  int* srow = sseq + ((B + 3) & ~3);
  // small batch: the whole table [B * MB]; else the range's window [kTblWin]
  const bool small = !MIX && p.dsmall != 0;
  int* tbl = sstart + ((B + 1 + 3) & ~3) + (MIX ? decode_mix_ints(B) : 0);
  char* slabs = reinterpret_cast<char*>(tbl + decode_tbl_ints(B, p.MB, small));
  __shared__ int wtot[8];

  KVS_PHASE(kPhaseStart);
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = hg * p.hpw + wave;
  W wv(p, g, slabs + wave * (C::SLAB + RB));
  if constexpr (ROPE) {
    wv.rcs = reinterpret_cast<float*>(slabs + wave * (C::SLAB + RB) + C::SLAB);
    if (lane < (p.rope_rd >> 1)) wv.theta = exp2(-(2.0 * lane / p.rope_rd) * p.rope_l2b);
  }
  typename W::NewRows nr;
  int Bn = B;   // sequences on the flattened axis
  if (small) {
    // ---- one memory round trip: this workgroup's first new rows (append),
    // seqlens_k and the whole block table; wave 0 forms the block prefix with
    // one in-register scan (B <= 64)
    if constexpr (SETUP_APPEND) nr = wv.append_fetch(w, nwg);
    const int L = wave == 0 && lane < B ? p.lens_k[lane] : 0;
    // the table in 16-byte pieces, kStageLoads per thread issued before any is
    // written (a write right after its own load would wait for that load,
    // making the staging one round trip per piece)
    const int nt = B * p.MB, nch = nt >> 2;
    auto stage = [&](int c0) __attribute__((always_inline)) {
      u32x4 v[kStageLoads];
#pragma unroll
      for (int k = 0; k < kStageLoads; ++k) {   // unconditional: pieces past the end re-read the last one
        const int c = c0 + k * nthr + tid;
        v[k] = ld16(p.table + 4 * min(c, nch - 1));
      }
#pragma unroll
      for (int k = 0; k < kStageLoads; ++k) {
        const int c = c0 + k * nthr + tid;
        if (c < nch) st16(tbl + 4 * c, v[k]);
      }
    };
    // the first batch outside any loop, so its loads are issued right behind
    // the length load (a loop would first wait for the loads before it)
    if (nch > 0) stage(0);
    for (int c0 = kStageLoads * nthr; c0 < nch; c0 += kStageLoads * nthr) stage(c0);
    for (int i = (nt & ~3) + tid; i < nt; i += nthr) tbl[i] = p.table[i];
    if (wave == 0) {
      const int nb = seq_blocks(L, win);
      const int x = wave_inclusive_sum(nb);
      if (lane < B) {
        slens[lane] = L;
        sstart[lane] = x - nb;
      }
      if (lane == B - 1) sstart[B] = x;
    }
    __syncthreads();
    KVS_PHASE(kPhaseStaged);
    if constexpr (SETUP_APPEND) wv.append_locate(nr, slens, tbl);
  } else {
    // ---- seqlens_k into LDS ---------------------------------------------------
    if constexpr (MIX) {
      // the one-row sequences, in batch order: a block-wide exclusive count
      // places each, with its query row and its key count
      const int per = (B + nthr - 1) / nthr;
      const int b0 = tid * per;
      int cnt = 0;
      for (int i = 0; i < per; ++i) {
        const int b = b0 + i;
        if (b < B && p.cu_q[b + 1] - p.cu_q[b] == 1) ++cnt;
      }
      const int x = wave_inclusive_sum(cnt);
      if (lane == 63) wtot[wave] = x;
      __syncthreads();
      int at = x - cnt;
      Bn = 0;
      for (int i = 0; i < nthr / 64; ++i) {
        if (i < wave) at += wtot[i];
        Bn += wtot[i];
      }
      for (int i = 0; i < per; ++i) {
        const int b = b0 + i;
        if (b < B) {
          const int q0 = p.cu_q[b];
          if (p.cu_q[b + 1] - q0 == 1) {
            sseq[at] = b;
            srow[at] = q0;
            slens[at] = p.lens_k[b];
            ++at;
          }
        }
      }
      Bn = __builtin_amdgcn_readfirstlane(Bn);
    } else {
      for (int b = tid; b < B; b += nthr) slens[b] = p.lens_k[b];
    }
    __syncthreads();

    // ---- exclusive prefix of the blocks per sequence over the batch, in LDS --
    {
      const int per = (Bn + nthr - 1) / nthr;
      const int b0 = tid * per;
      int run = 0;
      for (int i = 0; i < per; ++i) {
        const int b = b0 + i;
        if (b < Bn) run += seq_blocks(slens[b], win);
      }
      const int x = wave_inclusive_sum(run);
      if (lane == 63) wtot[wave] = x;
      __syncthreads();
      int base = 0;
      for (int i = 0; i < wave; ++i) base += wtot[i];
      int acc = base + x - run;
      for (int i = 0; i < per; ++i) {
        const int b = b0 + i;
        if (b < Bn) {
          sstart[b] = acc;
          acc += seq_blocks(slens[b], win);
        }
      }
      if (tid == nthr - 1) sstart[Bn] = acc;
      __syncthreads();
    }
    // append: this workgroup's first new rows are loaded now, with the table
    // window below, and stored once it has arrived
    if constexpr (SETUP_APPEND) nr = wv.append_load(w, nwg, slens);
  }
  KVS_PHASE(kPhasePrefix);
  const int total = sstart[Bn];
  const int r0 = (int)(((int64_t)w * total) / nwg), r1 = (int)(((int64_t)(w + 1) * total) / nwg);
  if (r0 >= r1) {  // empty range (whole workgroup)
    if constexpr (SETUP_APPEND) wv.append_rows(nr, w, nwg, slens);
    KVS_PHASE(kPhaseEnd);
    return;
  }

  auto seq_of = [&](int gb) __attribute__((always_inline)) {  // largest b with sstart[b] <= gb
    int lo = 0, hi = Bn - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sstart[mid] <= gb) lo = mid; else hi = mid - 1;
    }
    return lo;
  };

  // The range's table entries, once, in LDS (the planner keeps a range within
  // kTblWin blocks); a small batch has the whole table there already.
  if (!small) {
    for (int i = tid; i < r1 - r0; i += nthr) {
      const int gb = r0 + i;
      const int b = seq_of(gb);
      tbl[i] = p.table[(int64_t)(MIX ? sseq[b] : b) * p.MB + (gb - sstart[b]) + first_block(slens[b], win)];
    }
    __syncthreads();
  }
  KVS_PHASE(kPhaseWindow);
  if constexpr (SETUP_APPEND) wv.append_rows(nr, w, nwg, slens);
  KVS_PHASE(kPhaseNewRows);

  // Segments of the range, in processing order: the piece of the last sequence
  // Z (its head, unless it starts in this range), the piece of the first
  // sequence A (its tail), then the whole sequences in between.  The two
  // pieces that may be split come first, so they are published -- and their
  // sequences merged -- while other workgroups are still streaming.
  const int A = seq_of(r0), Z = seq_of(r1 - 1);
  const int nseg = A == Z ? 1 : 3;
  const int seg_lo0 = A == Z ? r0 : sstart[Z], seg_hi0 = r1;
  const int seg_lo1 = r0, seg_hi1 = A == Z ? r0 : sstart[A + 1];
  const int seg_lo2 = seg_hi1, seg_hi2 = A == Z ? r0 : sstart[Z];
  auto seg_lo = [&](int i) __attribute__((always_inline)) { return i == 0 ? seg_lo0 : (i == 1 ? seg_lo1 : seg_lo2); };
  auto seg_hi = [&](int i) __attribute__((always_inline)) { return i == 0 ? seg_hi0 : (i == 1 ? seg_hi1 : seg_hi2); };

  // split pieces: at most two (the pieces of Z and of A)
  int split_b0 = -1, split_n0 = 0, split_b1 = -1, split_n1 = 0;

  // step generator over segments [seg, seg_end): steps never cross a
  // sequence or a segment
  int seg = 0, seg_end = 0, pos = seg_lo0, sb = seq_of(seg_lo0);
  auto gen = [&]() __attribute__((always_inline)) {
    Step st;
    while (seg < seg_end && pos >= seg_hi(seg)) {
      ++seg;
      if (seg < seg_end) {
        pos = seg_lo(seg);
        if (pos < seg_hi(seg)) sb = seq_of(pos);
      }
    }
    if (seg >= seg_end) {
      st.b = -1; st.t = 0; st.Lk = 0; st.lblk = 0; st.nblk = 0; st.gblk = r0; st.first = 0; st.last = 0;
      return st;
    }
    while (sstart[sb + 1] <= pos) ++sb;
    const int s0 = sstart[sb], s1 = sstart[sb + 1];
    const int hi = seg_hi(seg);
    const int end = min(min(pos + C::NBS, s1), hi);
    st.b = sb;
    st.t = MIX ? srow[sb] : sb;   // (decode proper: cu_seqlens_q[b] = b)
    st.Lk = slens[sb];
    st.lblk = pos - s0 + first_block(st.Lk, win);
    st.nblk = end - pos;
    st.gblk = pos;
    st.first = pos == max(seg_lo(seg), s0) ? 1 : 0;
    st.last = end == min(hi, s1) ? 1 : 0;
    pos = end;
    return st;
  };
  auto phys_of = [&](const Step& st, int* ph) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < C::NBS; ++j)
      ph[j] = __builtin_amdgcn_readfirstlane(
          j < st.nblk ? tbl[small ? st.b * p.MB + st.lblk + j : st.gblk - r0 + j] : 0);
  };
  auto finish_piece = [&](const Step& st) __attribute__((always_inline)) {
    const int s0 = sstart[st.b], s1 = sstart[st.b + 1];
    const int a = max(r0, s0), z = min(r1, s1);
    if (a == s0 && z == s1) {
      wv.store_final(st.t);
    } else {
      // the first split piece is held and stored with the second (see
      // hold_partial); publish stores it if no second one comes
      if (split_b0 < 0) wv.hold_partial(w + st.b);
      else wv.store_partial(w + st.b);
      if (split_b0 < 0) {
        split_b0 = st.b;
        split_n0 = z - a;
      } else {
        split_b1 = st.b;
        split_n1 = z - a;
      }
    }
  };
  // Publish this wave's split pieces: count their blocks per (sequence, KV
  // head); the wave that completes a count merges that sequence's pieces.
  auto publish = [&]() __attribute__((always_inline)) {
    if (split_b0 < 0) return;
    wv.store_held();
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's partial stores are complete
    KVS_PHASE(kPhaseStores);
    // lane 0 counts the first split sequence, lane 1 the second: one atomic
    // instruction, one round trip
    const int mb = lane == 0 ? split_b0 : split_b1;
    const int mn = lane == 0 ? split_n0 : split_n1;
    bool done = false;
    if (lane < 2 && mb >= 0) {
      int* cnt = p.counters + (int64_t)mb * p.Hkv + g;
      const int need = sstart[mb + 1] - sstart[mb];
      done = __hip_atomic_fetch_add(cnt, mn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + mn == need;
      if (done) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
    }
    const uint64_t lastm = __ballot(done);
    KVS_PHASE(kPhaseCounters);
#ifdef KVS_PHASE_TIMES
    if (threadIdx.x == 0 && blockIdx.x < 4096) g_phase_t[blockIdx.x][kPhaseFlags] = lastm & 3;
#endif
    if (lastm & 3) {
      const int ba = (lastm & 1) ? split_b0 : split_b1;
      const int bb = (lastm & 3) == 3 ? split_b1 : ba;   // second sequence, if both are complete
      wv.merge((lastm & 3) == 3 ? 2 : 1, ba, MIX ? srow[ba] : ba, sstart[ba], sstart[ba + 1], bb, MIX ? srow[bb] : bb,
               sstart[bb], sstart[bb + 1], total, nwg);
    }
  };

  // Stream segments [s_begin, s_end) through the two-buffer pipeline.
  auto stream = [&](int s_begin, int s_end) __attribute__((always_inline)) {
    seg = s_begin;
    seg_end = s_end;
    pos = seg_lo(s_begin);
    if (pos < seg_hi(s_begin)) sb = seq_of(pos);
    if constexpr (BF16) {
      typename W::Buf bA, bB;
      int ph[C::NBS];
      Step cur = gen();
      if (cur.b < 0) return;
      phys_of(cur, ph);
      if constexpr (ROPE || (KV8 && APPEND)) cur.phys = ph[0];
      wv.load(cur, ph, bA);
      Step nxt = gen();
      for (;;) {
        phys_of(nxt, ph);
        if constexpr (ROPE || (KV8 && APPEND)) nxt.phys = ph[0];
        wv.load(nxt, ph, bB);
        if (cur.first) {
          wv.reset();
          if constexpr (ROPE) wv.rope_angles(cur.Lk);
        }
        wv.compute(cur, bA);
        if (cur.last) finish_piece(cur);
        cur = nxt;
        if (cur.b < 0) break;
        nxt = gen();
        phys_of(nxt, ph);
        if constexpr (ROPE || (KV8 && APPEND)) nxt.phys = ph[0];
        wv.load(nxt, ph, bA);
        if (cur.first) {
          wv.reset();
          if constexpr (ROPE) wv.rope_angles(cur.Lk);
        }
        wv.compute(cur, bB);
        if (cur.last) finish_piece(cur);
        cur = nxt;
        if (cur.b < 0) break;
        nxt = gen();
      }
    } else {
      int ph[C::NBS];
      for (Step cur = gen(); cur.b >= 0; cur = gen()) {
        phys_of(cur, ph);
        if (cur.first) wv.reset();
        wv.compute_f32(cur, ph);
        if (cur.last) finish_piece(cur);
      }
    }
  };

  // the pieces that may be split, then publish them, then the whole sequences
  const int nsplit_seg = nseg == 1 ? 1 : 2;
  stream(0, nsplit_seg);
  KVS_PHASE(kPhaseSplitDone);
  publish();
  KVS_PHASE(kPhaseMerged);
  if (nseg > nsplit_seg) stream(nsplit_seg, nseg);
  KVS_PHASE(kPhaseEnd);
}

template <int D, bool BF16, bool APPEND, bool WIN, bool KV8, bool ROPE, bool I8 = false>
__global__ __launch_bounds__(512) void decode_kernel(AttnParams p) {
  decode_body<D, BF16, APPEND, WIN, KV8, ROPE, I8>(p, (int)blockIdx.x, (int)blockIdx.y, p.nwg);
}

}  // namespace kvs
