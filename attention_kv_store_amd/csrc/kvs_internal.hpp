// Host/device shared parameter blocks and launcher declarations (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvs {

enum class DType : int { F32 = 0, BF16 = 1 };

struct StoreParams {
  const void* k_new;
  const void* v_new;
  const int32_t* slots;
  void* k_cache;
  void* v_cache;
  int64_t t_new;       // rows to store
  int64_t row_chunks;  // 16-byte chunks per token row (Hkv * D * esize / 16)
  int64_t num_slots;   // 16 * NB (only used by debug checks)
};

struct AttnParams {
  const void* q;          // [T, Hq, D]
  const void* k;          // [NB, 16, Hkv, D]
  const void* v;
  const int32_t* table;   // [B, MB]
  const int32_t* cu_q;    // [B + 1]
  const int32_t* lens_k;  // [B]
  void* out;              // [T, Hq, D]
  float* lse;             // [T, Hq] or null
  int32_t B, T, Hq, Hkv, MB;
  int32_t G;              // Hq / Hkv
  float scale_log2;       // scale * log2(e): scores are kept in base-2 units
  int32_t causal;
  // sliding window (needs causal): the row at position p sees keys
  // p - window + 1 .. p; 0 = no window
  int32_t window;
  // prefill work map
  int32_t HW;             // query heads per workgroup (divides G)
  int32_t TPW;            // 32-token blocks per workgroup (HW * TPW == 4 waves)
  int32_t NHG;            // head groups = Hq / HW
  int32_t pgrid;          // persistent workgroups
  int32_t pnw;            // waves per prefill workgroup (4: two per CU; 8: one per CU)
  int32_t meta_lds;       // 1: cu_seqlens_q and seqlens_k are staged in LDS
  // 1: every item index fits in 31 bits; items are then ordered per XCD and
  // decoded with multiply-high divisions (by NHG with the magic below)
  int32_t items32;
  uint32_t nhg_m, nhg_l;
  // decode work plan: the batch's key blocks, flattened sequence-major, are cut
  // into `nwg` equal contiguous ranges, one per workgroup; a workgroup holds the
  // waves of `hpw` consecutive KV heads.
  int32_t nwg;            // workgroups along the flattened block axis
  int32_t hpw;            // KV heads (waves) per workgroup
  float* part_o;          // [nwg + B, Hq, D] fp32 partial outputs (normalised)
  float* part_lse;        // [nwg + B, Hq]    fp32 partial lse (base 2)
  int32_t* counters;      // [B, Hkv]         finished-block counts; zero between calls
  // decode with append: the new K/V row of sequence b ([B, Hkv, D]) is its
  // key seqlens_k[b] - 1; it is read from here (not from the cache) and
  // written to the cache at that key's slot
  const void* k_new;
  const void* v_new;
  void* k_cache_w;
  void* v_cache_w;
  int32_t append;
  int32_t NB;             // cache blocks (the append writes only slots inside the pool)
  int32_t dsmall;         // decode: 1 = small batch, whole block table staged in LDS
  // FP8 (E4M3) caches: k / v hold codes, value = code * scale of its (slot, head)
  int32_t kv8;
  const float* k_scale;   // [NB, Hkv, 16]
  const float* v_scale;
  float* k_scale_w;       // FP8 fused decode step: the same scales, written at the new rows
  float* v_scale_w;
  // fused decode step with RoPE of q and the new key rows (position Lk - 1)
  int32_t rope;
  int32_t rope_rd;        // rotated dims per head
  int32_t rope_style;     // 0: pairs (i, i + rd/2); 1: pairs (2i, 2i + 1)
  double rope_inv_scale;  // 1 / pos_scale
  double rope_l2b;        // log2(base)
  // mixed launch (T != B): the first workgroups run the prefill items of the
  // sequences with more than one query row, the others the decode ranges of
  // the one-row sequences (split and merged as in decode); nwg is then the
  // capacity of the partial buffer, the decode ranges are formed in-kernel
  int32_t mixed;
};

// FP8 store: new rows [T, Hkv, D] (f32 / bf16) quantized into E4M3 code pools
// [NB, 16, Hkv, D] with one fp32 scale per (slot, head) in [NB, Hkv, 16].
struct StoreFp8Params {
  const void* k_new;
  const void* v_new;
  const int32_t* slots;
  void* k_cache;
  void* v_cache;
  float* k_scale;
  float* v_scale;
  int64_t t_new, num_slots;
  int32_t Hkv;
};

// RoPE + KV store: one workgroup per token row; angles from host-side
// frequencies theta_i = base^(-2 i / rd), i < rd / 2 <= kRopeMaxPairs.
constexpr int kRopeMaxPairs = 128;
struct RopeParams {
  void* q;                // [T, Hq, D], rotated in place (null: K/V only)
  const void* k_new;      // [T, Hkv, D]
  const void* v_new;
  const int32_t* pos;     // [T] positions
  const int32_t* slots;   // [T] pool slots (negative: row not stored)
  void* k_cache;          // [NB, 16, Hkv, D]
  void* v_cache;
  int64_t T, num_slots;
  int32_t Hq, Hkv, D;
  int32_t rd;             // rotated dims per head
  int32_t style;          // 0: pairs (i, i + rd/2); 1: pairs (2i, 2i + 1)
  double inv_scale;       // 1 / pos_scale
  double inv_freq[kRopeMaxPairs];
};

// Division by a divisor d (1 <= d < 2^31) fixed for a launch, for dividends
// n < 2^31: q = (mulhi(n, m) + n) >> l with l = ceil(log2 d) and
// m = floor(2^(32 + l) / d) - 2^32 + 1 (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994, section 4).
inline void fast_div_magic(uint32_t d, uint32_t* m, uint32_t* l) {
  uint32_t s = 0;
  while ((uint64_t(1) << s) < d) ++s;
  *l = s;
  *m = (uint32_t)(((uint64_t(1) << (32 + s)) / d) - (uint64_t(1) << 32) + 1);
}

// Split decode counts finished blocks per (sequence, KV head) in the first
// bytes of its workspace, at a place that does not depend on the shape.
constexpr size_t kDecodeCounterBytes = size_t(1) << 22;   // 2^20 counters

// Decode LDS bytes per workgroup: seqlens_k, block prefix, the table entries
// of the workgroup's range, then one V^T slab per wave.
constexpr int kDecodeTblWin = 2048;          // most blocks in one workgroup's range
// Small batches (B <= 64 and at most kDecodeSmallTbl table entries) stage the
// whole block table instead of a workgroup's window: one memory round trip
// then sets a workgroup up.
constexpr int kDecodeSmallB = 64;
constexpr int kDecodeSmallTbl = 16384;
__host__ __device__ inline int decode_tbl_ints(int B, int MB, bool small) { return small ? ((B * MB + 3) & ~3) : kDecodeTblWin; }
// the decode part of a mixed launch also keeps, per one-row sequence, its
// batch index and its query row
__host__ __device__ inline int decode_mix_ints(int B) { return 2 * ((B + 3) & ~3); }
inline size_t decode_lds_bytes(int B, int tbl_ints, int hpw, int slab_bytes) {
  const size_t ints = (size_t)((B + 3) & ~3) + (size_t)((B + 1 + 3) & ~3) + (size_t)tbl_ints;
  return ints * sizeof(int) + (size_t)hpw * slab_bytes;
}
// 16-key blocks per decode step over FP8 caches (bf16 / fp32: one).  Two
// blocks (the bf16 step's bytes in flight) measured slower than one: the FP8
// step is bounded by its instruction chain, not by the bytes it waits for.
constexpr int kDecodeKv8Blocks = 1;
// LDS bytes per decode wave: V^T, 16 keys (+ pad) x D per block of a step,
// then (fused RoPE step) the cos / sin of 64 angle pairs
constexpr int decode_slab_bytes(int D, bool kv8, bool rope = false) {
  return D * 40 * (kv8 ? kDecodeKv8Blocks : 1) + (rope ? 2 * 64 * 4 : 0);
}

// Prefill LDS bytes per workgroup: two K/V stages, then cu_seqlens_q and
// seqlens_k when staged.
inline size_t prefill_stage_bytes(int D, bool bf16) {
  // bf16: 64-key K and V tiles, unpadded rows; fp32: 32-key tiles, rows padded by 16 bytes
  return bf16 ? (size_t)2 * 64 * D * 2 : (size_t)2 * 32 * (D * 4 + 16);
}
// Prefill item order by decreasing work: batches of at most kSortB sequences
// whose workgroups have at most kSortRounds items each; the items of each
// round (pair and token tile) sit in LDS after the staged metadata.
constexpr int kSortB = 256;
constexpr int kSortRounds = 64;
inline size_t prefill_lds_bytes(int D, bool bf16, int B, int meta_lds) {
  const size_t meta = (size_t)(2 * B + 1) + (B <= kSortB ? 2 * kSortRounds : 0);
  return 2 * prefill_stage_bytes(D, bf16) + (meta_lds ? meta * sizeof(int) : 0);
}

// Device-side precondition check (debug library only): cu_seqlens_q (null:
// one row per sequence), seqlens_k, the table entries read, store slots.
struct CheckParams {
  const int32_t* cu_q;
  const int32_t* lens_k;
  const int32_t* table;
  int64_t B, T;
  int32_t MB, NB, window;
  const int32_t* slots;
  int64_t n_slots, num_slots;
};
enum { kCheckCuFirst = 1, kCheckCuLast = 2, kCheckLq = 3, kCheckLk = 4, kCheckTable = 5, kCheckSlot = 6 };
hipError_t run_check(const CheckParams& v, hipStream_t s, int out[4]);

hipError_t launch_store(const StoreParams& p, DType dt, hipStream_t s);
// zero `bytes` (a multiple of 16) at p, on stream s
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_rope_store(const RopeParams& p, DType dt, hipStream_t s);
// i8: INT8 codes (scale absmax / 127), else FP8 E4M3 (absmax / 448)
hipError_t launch_store_fp8(const StoreFp8Params& p, DType in, int D, bool i8, hipStream_t s);
hipError_t launch_prefill(const AttnParams& p, DType dt, int D, hipStream_t s);
hipError_t launch_decode(const AttnParams& p, DType dt, int D, hipStream_t s);
// mixed launch (bf16, 8-wave workgroups): `grid` workgroups, `lds` dynamic LDS bytes
hipError_t launch_mixed(const AttnParams& p, int D, int grid, size_t lds, hipStream_t s);

}  // namespace kvs
