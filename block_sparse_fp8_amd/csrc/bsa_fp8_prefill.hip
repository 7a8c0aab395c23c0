// Block-sparse FP8 (E4M3) attention prefill over a paged KV cache, gfx950.
//
// One workgroup of 256 threads (4 waves) owns one (sequence, q-head, 128-query
// tile); wave w owns queries 32w..32w+31, and each lane one query (S^T = K.Q^T
// puts a query in every accumulator column).  Two workgroups share a CU, so
// every SIMD runs two waves.
//
//   1. Active-tile compaction (hpc-ops article, "Active tile list"): each wave
//      ballots the Q tile's uint8 mask row 64 KV tiles at a time and walks the
//      set bits in ascending order, so every wave sees the same ordered list
//      without a round trip through LDS.  The candidates are clipped to the KV
//      length and, in causal mode, to the last tile any query of the Q tile can
//      see.  Tiles the mask switches off are never read.  In the index-list
//      form the same ballot runs over 64 list entries at a time (valid = a
//      tile id inside the candidate range) and the tile id is read from the
//      entry's lane, so tiles are visited in list order.
//   2. Per active tile, K, V and the per-token K descales go from the paged
//      cache straight to LDS (direct-to-LDS loads; a wave's 32 rows lie in one
//      page, so a whole tile needs one wave-uniform page base per wave).
//   3. S^T = K.Q^T on the E4M3 matrix path (v_mfma_f32_32x32x64_f8f6f4), by
//      default with two products per K operand.  These products sum 8
//      consecutive k at a time, each term aligned to the largest exponent sum
//      of the eight and cut below 2^-13 of it; so each query's codes are split
//      once between two operands, the codes within two binades of its largest
//      magnitude and the rest, which keeps small terms out of a group with a
//      large one (split_q).  Optionally one FP8 product per K operand (half
//      the matrix cycles, more bits lost), or f16 products
//      (v_mfma_f32_32x32x16_f16) on operands widened exactly (every E4M3
//      value, subnormals included, is an f16 normal): K once per workgroup
//      into an f16 tile, Q once in registers; they accumulate like fp32.  K
//      rows are read in a permuted order so that the accumulator registers of
//      lane half h hold keys h*32.. of each 64-key half of the tile, in
//      register order, the P operand's layout.
//   4. Online softmax in fp32 in the log2 domain: qscale*softmax_scale*log2(e)
//      (and the per-tensor K descale) is one per-lane constant; per-token K
//      descales multiply the scores.  P' = exp2(x - m + log2(p_scale)) =
//      p_scale*exp(score - max), so the P-scale (256 by default: hpc-ops
//      article, "FP8 Tensor Core compute: fixed P-scale quantisation"; any
//      p_scale in (0, 448]: "Quant Block Sparse Attention", "Key parameters")
//      costs nothing.  P' is rounded to E4M3 (v_cvt_pk_fp8_f32, round to
//      nearest even) and the row sum keeps the unrounded P'.
//   5. O^T += V^T . P^T on v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3).  V stays
//      row-major in LDS; the transposing read ds_read_b64_tr_b8 delivers it
//      key-major.
//   6. Epilogue: O = O_acc * vdescale / sum(P') (the 1/p_scale is inside the
//      sum), written as bf16; LSE = ln2 * (m + log2(sum) - log2(p_scale)).  A
//      query whose sparse set is empty gets O = 0 and LSE = -FLT_MAX ("Quant
//      Block Sparse Attention", "Sparse indices & PA page table").
//
// The tile loop is software-pipelined inside each wave (see the comment above
// the kernel): the products of the next tile's scores run among the current
// tile's exponentials, and the next tile's maximum among the current tile's
// P.V products, so that one wave keeps the matrix pipe and the VALU busy.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>
#include <math.h>
#include <string.h>

#include "bsa_fp8.h"
#include "bsa_internal.h"

namespace {

using bsa::kTile;
using bsa::kHeadDim;
using bsa::kFormList;
using bsa::candidate_end;
constexpr int kThreads = 256;
constexpr int kK16Row = 2 * kHeadDim;  // bytes per f16 K row in LDS
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegFltMax = -3.402823466e+38f;

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

struct Params {
  const uint8_t* q;
  const uint8_t* kc;
  const uint8_t* vc;
  const float* qscale;
  const float* kscale;
  const float* vscale;
  const int32_t* cu_q;
  const int32_t* block_table;
  const int32_t* seqlens_kv;
  const uint8_t* mask;
  const int32_t* sidx;      // index-list form: [B, Hq, mt, mkv] tile ids
  const int32_t* slen;      // index-list form: [B, Hq, mt] valid lengths
  const int32_t* schedule;  // task order, or nullptr for the built-in order
  uint16_t* out;
  float* lse;
  int B, T, Hq, Hkv, group;
  int page_size, page_shift, max_pages;
  int mt, mkv, mt_grid;
  int layout, causal;
  float qk_scale;       // softmax_scale * log2(e)
  float pscale_log2;    // log2(p_scale)
  int q_tok_stride;     // q rows (of 128 B) between consecutive tokens: Hq (TND) or 1 (NTD)
  int q_head_stride;    // q rows between consecutive heads: 1 (TND) or T (NTD)
  uint32_t page_bytes;  // bytes of one page of K (or V) cache: page_size * Hkv * 128
  int slot_stride;      // rows between consecutive slots of a page (Hkv for NHD, 1 for HND)
  int head_stride;      // rows between consecutive kv-heads of a page (1 for NHD, page_size for HND)
};

// 16-byte chunk swizzle of the E4M3 K and V rows (128 B, 8 chunks) in LDS:
// chunk c of row r sits at c ^ (r & 7) ^ bit 5 of r.  Both read patterns are
// then free of bank conflicts: the transposing V reads, and the FP8 K operand
// reads, whose 16 lanes per pass take rows r0+{0..3, 4..7, 32..35, 36..39}.
__device__ __forceinline__ int swz8(int row) { return (row & 7) ^ ((row >> 5) & 1); }


__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Four E4M3 codes (one dword) -> four f16 values, exactly (every E4M3 value,
// subnormals included, is an f16 normal).  Returned as two dwords.
__device__ __forceinline__ v2i e4m3x4_to_f16x4(uint32_t w) {
  const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
  return v2i{(int)lo, (int)hi};
}

__device__ __forceinline__ v16f mfma_f8(v8i a, v8i b, v16f c) {
  // E4M3 (format 0) for both operands, no block scales.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v16f mfma_f16(v8h a, v8h b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// Wave-uniform walk over the active KV tiles of one Q tile, in ascending order.
struct MaskWalk {
  const uint8_t* row;  // mask row, or nullptr for the dense path
  int n_end;           // candidates are 0 .. n_end-1
  int base;            // first candidate of the current 64-tile chunk
  uint64_t bits;       // active candidates of the chunk not yet returned

  __device__ void init(const uint8_t* r, int end, int lane) {
    row = r;
    n_end = end;
    base = 0;
    bits = load_chunk(lane);
  }
  __device__ uint64_t load_chunk(int lane) const {
    int n = base + lane;
    asm volatile("" : "+v"(n));  // no per-lane pointer kept live across the tile loop
    const bool act = n < n_end && (row == nullptr || row[n] != 0);
    return __ballot(act);
  }
  // Next active tile, or -1.
  __device__ int next(int lane) {
    while (bits == 0) {
      base += 64;
      if (base >= n_end) return -1;
      bits = load_chunk(lane);
    }
    const int n = base + (int)__builtin_ctzll(bits);
    bits &= bits - 1;
    return n;
  }
};

// Wave-uniform walk over an index list, in list order.  Entries outside
// [0, n_end) select no key any query of the Q tile may see and are skipped.
struct ListWalk {
  const int32_t* row;  // the Q tile's list
  int len;             // valid entries: 0 .. len-1
  int n_end;           // candidate tiles are 0 .. n_end-1
  int base;            // first entry of the current 64-entry chunk
  uint64_t bits;       // usable entries of the chunk not yet returned
  int ent;             // this lane's entry of the chunk

  __device__ void init(const int32_t* r, int length, int end, int lane) {
    row = r;
    len = length;
    n_end = end;
    base = 0;
    bits = len > 0 ? load_chunk(lane) : 0;
  }
  __device__ uint64_t load_chunk(int lane) {
    int i = base + lane;
    asm volatile("" : "+v"(i));
    ent = i < len ? row[i] : -1;
    return __ballot(ent >= 0 && ent < n_end);
  }
  __device__ int next(int lane) {
    while (bits == 0) {
      base += 64;
      if (base >= len) return -1;
      bits = load_chunk(lane);
    }
    const int pos = (int)__builtin_ctzll(bits);
    bits &= bits - 1;
    return __builtin_amdgcn_readlane(ent, pos);
  }
};

// Direct-to-LDS loads, issued through asm so that the compiler does not make
// LDS reads of other buffers wait for them (every one is waited for
// explicitly, by `s_waitcnt vmcnt(0)` before the barrier that publishes its
// data).  A wave writes 64 consecutive elements (16 or 4 bytes per lane) at
// the wave-uniform LDS address `lds`.  M0 is set here and used by nothing
// else in the kernel.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory");
}
// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane offset.
__device__ __forceinline__ void dma16s(uint32_t off, uint64_t sbase, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(sbase), "s"(lds) : "memory");
}
__device__ __forceinline__ void dma4s(uint32_t off, uint64_t sbase, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(sbase), "s"(lds) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// Matrix paths of the Q.K^T products (template argument of the kernel).
constexpr int kQkF16 = 0;       // E4M3 widened exactly to f16, f16 products
constexpr int kQkFp8 = 1;       // E4M3 operands, one FP8 product per K operand
constexpr int kQkFp8Split = 2;  // E4M3 operands, two FP8 products per K operand

// Magnitude split of a query's E4M3 codes between two FP8 products.
// The FP8 products sum 8 consecutive k at a time, each term aligned to the
// largest exponent sum of the eight and cut below 2^-13 of it, so small terms
// beside a large one lose bits.  Codes within two binades of the query's
// largest magnitude (magnitude code >= max - 16) stay in `a`; the others move
// to `b`, and each position holds its code in exactly one of the two (+0 in
// the other), so the two products sum to the same dot product.  A lane holds
// half of its query's dims and lane l ^ 32 the other half, so the maximum is
// taken over both.  E4M3 magnitudes order like their 7-bit codes, so the test
// is a byte compare.
__device__ __forceinline__ void split_q(v8i* a, v8i* b) {
  uint32_t mx = 0;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t m = (uint32_t)a[ks][i] & 0x7f7f7f7fu;
      mx = max(mx, max(max(m & 0xffu, (m >> 8) & 0xffu), max((m >> 16) & 0xffu, m >> 24)));
    }
  const auto sw = __builtin_amdgcn_permlane32_swap(mx, mx, false, false);
  mx = max(sw[0], sw[1]);
  const uint32_t thr = mx > 16u ? mx - 16u : 0u;
  const uint32_t add = (0x80u - thr) * 0x01010101u;  // bit 7 of a byte set iff its magnitude >= thr
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w = (uint32_t)a[ks][i];
      const uint32_t sel = ((w & 0x7f7f7f7fu) + add) & 0x80808080u;
      const uint32_t keep = sel | (sel - (sel >> 7));  // 0xff where selected
      a[ks][i] = (int)(w & keep);
      b[ks][i] = (int)(w & ~keep);
    }
}

// The software-pipelined tile loop.  Per active tile t (with t1, t2 the next
// two) each wave runs two phases whose matrix products and VALU work are
// independent, so that one wave keeps both the matrix pipe and the VALU busy:
//   A: exponentials, E4M3 packs and row sums of S(t) (scaled and max-reduced
//      in the previous step), interleaved block by block with the products of
//      S(t1) = K(t1).Q^T; the registers of S(t) are freed as those of S(t1)
//      fill.
//   B: O *= alpha(t) and O += V(t)^T.P(t)^T, interleaved with the K descales,
//      band mask and row maximum of S(t1), and (f16 products) the widening of
//      K(t2) into the f16 tile.
// Loads of a step (V(t), the K descales of t1, the raw K of t2, the page ids
// of the tile after t2) are issued at its start and waited for before the
// barrier that separates A from B.
template <int QUANT, int FORM, int QKM>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
bsa_fp8_prefill_kernel(Params p) {
  constexpr bool QK8 = QKM != kQkF16;          // E4M3 operands on the FP8 products
  constexpr bool SPLIT = QKM == kQkFp8Split;   // two products per K operand (split Q)
  // K for the products: f16 chunk-major tile (32 KB: 16-byte chunk c, dims
  // 8c..8c+7, of key row r at c*2048 + r*16) fed from an E4M3 staging tile; or
  // (FP8 products) a ring of two E4M3 tiles.  E4M3 tiles are row-major with
  // the 16-byte chunks of row r permuted by swz8(r).
  constexpr int kKBytes = QK8 ? 2 * kTile * kHeadDim : kTile * kK16Row;
  __shared__ __attribute__((aligned(16))) uint8_t kmat_lds[kKBytes];
  __shared__ __attribute__((aligned(16))) uint8_t kst_lds[QK8 ? 16 : kTile * kHeadDim];
  // V and the K descales: on the FP8 paths two buffers each (step parity), so
  // that a step needs one barrier; the f16 path has room for one of each.
  // After the descale buffers, one region of 1.0 (see the band tiles in the
  // tile loop).
  constexpr int kVBufs = QK8 ? 2 : 1;
  constexpr int kOnes = kVBufs;  // descale slot that holds 1.0 for every key
  __shared__ __attribute__((aligned(16))) uint8_t v8_lds[kVBufs * kTile * kHeadDim];
  __shared__ __attribute__((aligned(16))) float ks_lds[(kVBufs + 1) * kTile];
  // FP8 paths: each lane's LDS read offsets, written once: the four K operand
  // chunks of a block (two 16-byte chunks for each of the two 64-dim steps)
  // and the four V operand columns of a 64-key step.  A step reads them back
  // with two LDS loads instead of deriving them from the lane id again (which
  // the loop cannot keep in registers).
  __shared__ __attribute__((aligned(16))) int ofs_lds[QK8 ? kThreads * 8 : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hd = lane >> 5;   // lane half
  const int col = lane & 31;  // query column owned by this lane within the wave

  // LDS read offsets of lane ln within an E4M3 tile (FP8 paths: computed once
  // and kept in ofs_lds; the f16 path derives the V offsets where it reads).
  // K operand of the Q.K^T products: for the 64-dim step ks, the lane reads
  // logical chunks 4ks + 2*(ln >> 5) and the next one of key row row0 (plus a
  // per-block constant row offset, see kop).  Entry 2ks + h is chunk h.
  auto k_offsets = [](int ln) -> v4i {
    const int lcol = ln & 31;
    const int row0 = ((lcol >> 2) & 1) * 32 + (((lcol >> 3) << 2) | (lcol & 3));
    const int sw = swz8(row0);
    const int c0 = 2 * (ln >> 5);
    return v4i{row0 * kHeadDim + ((c0 ^ sw) << 4), row0 * kHeadDim + (((c0 + 1) ^ sw) << 4),
               row0 * kHeadDim + (((c0 + 4) ^ sw) << 4), row0 * kHeadDim + (((c0 + 5) ^ sw) << 4)};
  };
  // V operand of the P.V products (transposing read): in each 16-lane group,
  // source lane 2k+q addresses key row (half*32 + 8*rr + k) of a 64-key step
  // at head-dim column 32d + 16*(group & 1) + 8q; result lane i then holds
  // that column + i for those 8 keys.  The rows half*32 + 8*rr + k share the
  // lane's chunk swizzle, so the offset for output block d serves every rr
  // and both 64-key steps through constant offsets.
  auto v_offset = [](int ln, int d) -> int {
    const int grp = ln >> 4;
    const int kk = (ln & 15) >> 1;
    const int half = grp >> 1;
    const int csw = (grp & 1) ^ kk ^ half;  // logical chunk 2d + (grp&1), swizzled
    return (half * 32 + kk) * kHeadDim + 8 * (ln & 1) + (((2 * d) ^ csw) << 4);
  };
  if (tid < kTile) ks_lds[kOnes * kTile + tid] = 1.0f;
  if constexpr (QK8) {
    *reinterpret_cast<v4i*>(&ofs_lds[tid * 8]) = k_offsets(lane);
    *reinterpret_cast<v4i*>(&ofs_lds[tid * 8 + 4]) =
        v4i{v_offset(lane, 0), v_offset(lane, 1), v_offset(lane, 2), v_offset(lane, 3)};
  }

  // Work order.  The hardware hands consecutive workgroup ids to the 8 XCDs
  // round-robin.  Without a schedule, id i is remapped so that XCD (i % 8)
  // walks its own share of the tasks (below); when Hq is not a multiple of 8
  // the share is a contiguous slice of the list ordered by kv-group (kv-head
  // outer, sequence inner), then Q tile from the last down, then q-head within
  // the group.  Each XCD's L2 then serves the K/V of its own kv-heads.
  // A schedule (from the pre-pass) names the task directly: task id
  // (b * Hq + h) * mt_grid + m.
  const int total = p.B * p.Hq * p.mt_grid;
  int m, b, h, g;
  if (p.schedule != nullptr) {
    const int task = p.schedule[blockIdx.x];
    if ((unsigned)task >= (unsigned)total) return;  // not a task id: nothing to do
    m = task % p.mt_grid;
    const int bh = task / p.mt_grid;
    h = bh % p.Hq;
    b = bh / p.Hq;
    g = h / p.group;
  } else if ((p.Hq & 7) == 0) {
    // Workgroup i runs on XCD i % 8.  XCD x owns q-heads [x*Hq/8, (x+1)*Hq/8),
    // every sequence and Q tile of them, so the eight shares have the same
    // shape and a kv-head's K/V stays within one or two XCDs' L2.  Within a
    // share: sequence, then Q tile from the last (most causal work) down, then
    // head.
    const int x = (int)(blockIdx.x & 7);
    const int r = (int)(blockIdx.x >> 3);
    const int hpx = p.Hq >> 3;
    const int q = r / hpx;
    h = x * hpx + (r - q * hpx);
    m = p.mt_grid - 1 - q % p.mt_grid;
    b = q / p.mt_grid;
    g = h / p.group;
  } else {
    const int per_xcd = total >> 3;
    const int i = (int)blockIdx.x;
    const int L = i < (per_xcd << 3) ? (i & 7) * per_xcd + (i >> 3) : i;
    const int per_group = p.group * p.mt_grid;
    const int gi = L / per_group;
    const int within = L - gi * per_group;
    m = p.mt_grid - 1 - within / p.group;
    b = gi % p.B;
    g = gi / p.B;
    h = g * p.group + within % p.group;
  }

  const int t0 = p.cu_q[b];
  const int lq = p.cu_q[b + 1] - t0;
  const int lkv = p.seqlens_kv[b];
  if (m * kTile >= lq) return;  // Q tile beyond this sequence (uniform per workgroup)

  // Candidate KV tiles: below the KV length, within the causal range of some
  // query of this Q tile, and (mask form) within the mask width.
  int n_end = candidate_end(lq, lkv, m, p.causal);
  const int64_t qrow = ((int64_t)b * p.Hq + h) * p.mt + m;  // row of the sparsity arrays
  std::conditional_t<FORM == kFormList, ListWalk, MaskWalk> walk;
  if constexpr (FORM == kFormList) {
    const int len = min(max(p.slen[qrow], 0), p.mkv);
    walk.init(p.sidx + qrow * p.mkv, len, n_end, lane);
  } else {
    const uint8_t* mask_row = nullptr;
    if (p.mask != nullptr) {
      n_end = min(n_end, p.mkv);
      mask_row = p.mask + qrow * p.mkv;
    }
    walk.init(mask_row, n_end, lane);
  }

  // Queries of this lane.
  const int tq = m * kTile + wave * 32 + col;             // query index within the sequence
  const bool q_valid = tq < lq;
  const int p_wave_min = lkv - lq + m * kTile + wave * 32;  // smallest position in the wave

  // Q operand (B of S^T = K.Q^T): f16 products, lane holds query `col`,
  // head-dim elements ks*16 + hd*8 .. +7 for ks = 0..7; FP8 products, dims
  // ks*64 + hd*32 .. +31 for ks = 0..1.
  v8h qh[QK8 ? 1 : 8];
  v8i q8[QK8 ? 2 : 1];
  v8i q8b[SPLIT ? 2 : 1];  // split products: the codes of the second product
  v2i qraw[QK8 ? 1 : 8];
  float cscale = 0.0f;
  {
    const int64_t qi = (int64_t)(t0 + (q_valid ? tq : 0)) * p.q_tok_stride + (int64_t)h * p.q_head_stride;
    if constexpr (QK8) {
      const uint8_t* qp = p.q + qi * kHeadDim + hd * 32;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        q8[ks] = q_valid ? *reinterpret_cast<const v8i*>(qp + ks * 64) : v8i{0, 0, 0, 0, 0, 0, 0, 0};
    } else {
      const uint8_t* qp = p.q + qi * kHeadDim + hd * 8;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qraw[ks] = q_valid ? *reinterpret_cast<const v2i*>(qp + ks * 16) : v2i{0, 0};
    }
    if (q_valid) cscale = p.qscale[qi] * p.qk_scale;
  }
  if constexpr (SPLIT) split_q(q8, q8b);
  auto widen_q = [&]() {
    if constexpr (!QK8) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const v2i a = e4m3x4_to_f16x4((uint32_t)qraw[ks][0]);
        const v2i c = e4m3x4_to_f16x4((uint32_t)qraw[ks][1]);
        qh[ks] = __builtin_bit_cast(v8h, v4i{a[0], a[1], c[0], c[1]});
      }
    }
  };
  if (QUANT == BSA_QUANT_Q_TOKHEAD_K_TENSOR_V_TENSOR) cscale *= p.kscale[0];
  // Keep the score constant strictly positive so that a masked score (-inf)
  // maps to exp2(-inf) = 0 without a select.  Descales are >= 0 and the
  // softmax scale is >= 0 (the host refuses a negative one), so this only
  // changes a zero constant, where every x is then ~1e-38 * S instead of 0.
  cscale = fmaxf(cscale, 1.17549435e-38f);

  v16f oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[d][r] = 0.0f;
  float m_run = -INFINITY;  // running max of x = score * log2(e)
  float l_run = 0.0f;       // this lane's half of sum(P'), P' = p_scale * 2^(x - m)
  float alpha = 0.0f;       // rescale of O before the next P.V
  float bias = 0.0f;        // log2(p_scale) - m for the exponentials
  bool rescale = false;     // some row of the wave has a new maximum

  // ---- addresses ------------------------------------------------------------
  const int32_t* bt = p.block_table + (int64_t)b * p.max_pages;
  const int head_row = g * p.head_stride;
  const int pmask = p.page_size - 1;
  // Byte offset of (page, slot, this kv-head) in a cache: one 32x32->64-bit
  // product per page plus 32-bit in-page arithmetic.
  auto row_addr = [&](const uint8_t* base, int pg, int slot) -> const uint8_t* {
    return base + (uint64_t)(uint32_t)pg * p.page_bytes + (uint32_t)(slot * p.slot_stride + head_row) * kHeadDim;
  };
  // Page id of tile n for this wave: the 32 rows a wave loads (K, V and the
  // K descales) lie in one 32-aligned block, hence in one page.  The row is
  // clamped to lkv-1, so no block-table entry past the sequence's pages is
  // read.  (An opaque zero in a vector register keeps the lookup a per-lane
  // load: a wave-uniform one would be moved to a scalar register at once,
  // whose wait also waits for every load in flight; the value moves to a
  // scalar register once it has arrived.  The zero is made afresh for each
  // lookup so that no register holds it across the loop.)
  struct Pages {
    int kv;
  };
  auto lookup = [&](int n, int ln) -> Pages {
    (void)ln;
    int vzero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));
    Pages ps;
    ps.kv = bt[min(n * kTile + wave * 32 + vzero, lkv - 1) >> p.page_shift];
    return ps;
  };
  // One E4M3 tile (K or V) of tile n into LDS at `dst` (row-major, chunks
  // permuted by swz8): wave w loads rows 32w..32w+31, 8 rows of 128 bytes per
  // instruction.  Rows past the KV length read row lkv-1 (finite; their P is 0).
  // A whole tile inside the KV length: the wave's 32 rows are consecutive
  // slots of one page, and since 128 is a multiple of the page size, every
  // lane's offset within the page (its slot, the kv-head and its swizzled
  // chunk) is the same for every tile: only the page base changes, a
  // wave-uniform value in SGPRs.
  const int drow = wave * 32 + (lane >> 3);  // tile row of the lane's first load
  const uint32_t dma_off =
      (uint32_t)((drow & pmask) * p.slot_stride + head_row) * kHeadDim + (uint32_t)(((lane & 7) ^ swz8(drow)) << 4);
  const uint64_t dma_step = 8ull * (uint64_t)p.slot_stride * kHeadDim;  // 8 rows further
  auto dma_tile = [&](const uint8_t* cache, int n, int pg, uint8_t* dst, int ln) {
    const int row0 = wave * 32 + (ln >> 3);
    const uint32_t base = lds_addr(dst) + (uint32_t)(wave * 32) * kHeadDim;
    if (n * kTile + kTile <= lkv) {
      const uint64_t sbase =
          (uint64_t)(uintptr_t)cache + (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(pg) * p.page_bytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) dma16s(dma_off, sbase + i * dma_step, base + i * 8 * kHeadDim);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = row0 + i * 8;
        const int j = min(n * kTile + row, lkv - 1);
        dma16(row_addr(cache, pg, j & pmask) + (((ln & 7) ^ swz8(row)) << 4), base + i * 8 * kHeadDim);
      }
    }
  };
  // The K descales of the wave's 32 rows (lanes 0..31, one float each) from
  // the same page: the descale array is laid out like the cache without the
  // head dimension.  Rows past the KV length read row lkv-1.
  auto dma_kscale = [&](int n, int pg, int ln, int slot) {
    if (QUANT == BSA_QUANT_Q_TOKHEAD_K_TOKHEAD_V_HEAD) {
      const int row = n * kTile + wave * 32 + (ln & 31);
      const uint32_t off = (uint32_t)((min(row, lkv - 1) & pmask) * p.slot_stride + head_row) * 4u;
      const uint64_t sbase = (uint64_t)(uintptr_t)p.kscale +
                             (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(pg) * (p.page_bytes / kHeadDim) * 4u;
      if (ln < 32) dma4s(off, sbase, lds_addr(ks_lds + slot * kTile) + wave * 32 * 4);
    }
  };
  // f16 products: widen the staged E4M3 K tile into the f16 tile.  Thread
  // (row tid & 127, half tid >> 7) converts dims 64*half .. +63 of its row.
  // `part` (0..3) selects one 16-byte chunk of the thread's four.
  auto widen_k = [&](int part, int ln) {
    if constexpr (!QK8) {
      const int r = (wave & 1) * 64 + ln;
      const int half = wave >> 1;
      const uint8_t* src = kst_lds + r * kHeadDim;
      {
        const int c8 = 4 * half + part;  // logical E4M3 chunk: dims 16*c8 .. +15
        const v4i w = *reinterpret_cast<const v4i*>(src + ((c8 ^ swz8(r)) << 4));
        const v2i a = e4m3x4_to_f16x4((uint32_t)w[0]);
        const v2i c = e4m3x4_to_f16x4((uint32_t)w[1]);
        const v2i d = e4m3x4_to_f16x4((uint32_t)w[2]);
        const v2i e = e4m3x4_to_f16x4((uint32_t)w[3]);
        *reinterpret_cast<v4i*>(kmat_lds + (2 * c8) * 2048 + r * 16) = v4i{a[0], a[1], c[0], c[1]};
        *reinterpret_cast<v4i*>(kmat_lds + (2 * c8 + 1) * 2048 + r * 16) = v4i{d[0], d[1], e[0], e[1]};
      }
    }
  };

  // ---- the products S^T = K.Q^T -------------------------------------------------
  // Accumulator row i of block c holds key (c>>1)*64 + hi*32 + (c&1)*16 + ri,
  // hi = (i>>2)&1, ri = (i>>3)*4 + (i&3): the lane of half h then holds keys
  // (c>>1)*64 + h*32 + (c&1)*16 + 0..15 in register order, the layout the P
  // operand of P.V needs.  Product j of a tile is block j / kPerBlock, k-step
  // j % kPerBlock; kop(j) reads its K operand.
  constexpr int kPerBlock = QK8 ? 2 : 8;          // products per 32-key block
  // K operand reads ahead of their product (each split operand feeds two)
  constexpr int kAhead = SPLIT ? 1 : (QK8 ? 2 : 3);
  using KOp = std::conditional_t<QK8, v8i, v8h>;
  // Lane ln's key row within block c is (c >> 1) * 64 + (c & 1) * 16 + row0,
  // row0 = 32 * bit 2 of the query column + (bits 3, 1, 0 of it); the block's
  // rows share row0's chunk swizzle (bits 0-2 and 5 of the row), so on the
  // FP8 paths the block only adds a constant to the lane's four offsets `ko`
  // (from k_offsets).
  auto kop = [&](int j, int ln, const v4i& ko, const uint8_t* kbuf) -> KOp {
    const int c = j / kPerBlock, ks = j % kPerBlock;
    if constexpr (QK8) {
      const uint8_t* kp = kbuf + ((c >> 1) * 64 + (c & 1) * 16) * kHeadDim;
      const v4i lo = *reinterpret_cast<const v4i*>(kp + ko[2 * ks]);
      const v4i hi = *reinterpret_cast<const v4i*>(kp + ko[2 * ks + 1]);
      return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      const int lcol = ln & 31;
      const int row = (c >> 1) * 64 + ((lcol >> 2) & 1) * 32 + (c & 1) * 16 + (((lcol >> 3) << 2) | (lcol & 3));
      return *reinterpret_cast<const v8h*>(kmat_lds + (ln >> 5) * 2048 + row * 16 + ks * 4096);
    }
  };
  auto mfma_qk = [&](const KOp& a, int ks, const v16f& acc) -> v16f {
    if constexpr (SPLIT) return mfma_f8(a, q8b[ks], mfma_f8(a, q8[ks], acc));
    else if constexpr (QK8) return mfma_f8(a, q8[ks], acc);
    else return mfma_f16(a, qh[ks], acc);
  };
  // All four blocks of a tile with no other work (the prologue).
  auto qk_tile = [&](v16f* out, int ln, const v4i& ko, const uint8_t* kbuf) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v16f acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < kPerBlock; ++ks) acc = mfma_qk(kop(c * kPerBlock + ks, ln, ko, kbuf), ks, acc);
      out[c] = acc;
    }
  };

  // ---- per-block softmax pieces ------------------------------------------------
  // The K descales of block c (per-token K scales), read ahead of their use;
  // slot kOnes reads 1.0 for every key.
  auto ks_read = [&](int c, int ln, int slot) -> v16f {
    v16f k;
    if (QUANT == BSA_QUANT_Q_TOKHEAD_K_TOKHEAD_V_HEAD) {
      const float* ksp = &ks_lds[slot * kTile + (c >> 1) * 64 + (ln >> 5) * 32 + (c & 1) * 16];
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const v4f t = *reinterpret_cast<const v4f*>(ksp + r);
        k[r] = t[0];
        k[r + 1] = t[1];
        k[r + 2] = t[2];
        k[r + 3] = t[3];
      }
    }
    return k;
  };
  // Whether tile n reaches past a query of the wave (causal) or past the KV
  // length, i.e. needs the band mask.
  auto band_tile = [&](int n) -> bool {
    return (p.causal && n * kTile + kTile - 1 > p_wave_min) || (n * kTile + kTile > lkv);
  };
  // Band mask of block c of tile n, in place.
  auto mask_block = [&](v16f& sb, int c, int n, int ln) {
    const int lhd = ln >> 5;
    const int lcol = ln & 31;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = n * kTile + (c >> 1) * 64 + lhd * 32 + (c & 1) * 16 + r;
      const bool ok = j < lkv && (!p.causal || j <= p_wave_min + lcol);
      sb[r] = ok ? sb[r] : -INFINITY;
    }
  };
  // K descales of one block of S (in place).
  auto scale_block = [&](v16f& sb, const v16f& kd) {
    if (QUANT == BSA_QUANT_Q_TOKHEAD_K_TOKHEAD_V_HEAD) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sb[r] *= kd[r];
    }
  };
  // The block's partial maximum of the unscaled-by-cscale score, folded with
  // run_max.
  auto max_block = [&](const v16f& sb, float run_max) -> float {
    const float a = max3f(max3f(sb[0], sb[1], sb[2]), max3f(sb[3], sb[4], sb[5]), max3f(sb[6], sb[7], sb[8]));
    const float b2 = max3f(max3f(sb[9], sb[10], sb[11]), max3f(sb[12], sb[13], sb[14]), sb[15]);
    return max3f(a, b2, run_max);
  };
  // Scale + band mask + maximum of one block of S of tile n (in place).
  auto prep_block = [&](v16f& sb, const v16f& kd, int c, int n, int ln, float run_max) -> float {
    scale_block(sb, kd);
    if (band_tile(n)) mask_block(sb, c, n, ln);
    return max_block(sb, run_max);
  };
  // New running maximum from the four blocks' partial maxima (both lane
  // halves): sets alpha, bias and rescale.
  auto update_max = [&](float tmax) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
    tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    const float tmax_x = tmax == -INFINITY ? -INFINITY : tmax * cscale;
    const float m_new = fmaxf(m_run, tmax_x);
    const float m_safe = m_new == -INFINITY ? 0.0f : m_new;
    alpha = __builtin_amdgcn_exp2f(m_run - m_safe);  // exp2(-inf) = 0
    bias = p.pscale_log2 - m_safe;
    rescale = __ballot(m_new != m_run) != 0;
    m_run = m_new;
  };
  // P' = exp2(s*cscale + bias) of one block: its partial row sum, and its
  // E4M3 codes into the P operand (bytes (c&1)*16 + r of P.V step c>>1).
  // Masked scores are -inf and cscale > 0, so their P' is exactly 0.
  auto exp_block = [&](const v16f& sb, int c, v8i* pk) -> float {
    float ls = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r += 4) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(sb[r], cscale, bias));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(sb[r + 1], cscale, bias));
      const float e2 = __builtin_amdgcn_exp2f(fmaf(sb[r + 2], cscale, bias));
      const float e3 = __builtin_amdgcn_exp2f(fmaf(sb[r + 3], cscale, bias));
      ls += (e0 + e1) + (e2 + e3);
      // (the first pack's high half is replaced by the second: any old value
      // serves, and on the FP8 paths e0's register, free by then, saves a
      // zeroing move; the f16 path has no register to spare for it)
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, QK8 ? __float_as_int(e0) : 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, w, true);
      pk[c >> 1][(c & 1) * 4 + (r >> 2)] = w;
    }
    return ls;
  };

  // O^T += V^T . P^T for 32 output dims (block d), both 64-key steps; on the
  // FP8 paths `vo` holds the lane's four v_offset values.
  auto vread = [&](int x, int ln, const v4i& vo, int slot) -> v8i {  // x = sp*4 + d
    const int vof = QK8 ? vo[x & 3] : v_offset(ln, x & 3);
    const uint8_t* vp = v8_lds + slot * kTile * kHeadDim + vof + (x >> 2) * 64 * kHeadDim;
    v8i a;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vp + rr * 8 * kHeadDim));
      a[2 * rr] = t[0];
      a[2 * rr + 1] = t[1];
    }
    return a;
  };

  // ---- the tile list ------------------------------------------------------------
  // n: tile of the current step (its S is ready); n1, n2: the next two; n3 is
  // looked up during the step.  Page ids: pg_n for n (V), pg_1 for n1 (K
  // descales), pg_2 for n2 (K), pg_3 for n3.
  // The stores at the end derive the lane's query and half again from a
  // fresh lane id (an opaque instruction, not a copy of `lane`), so that
  // neither stays live, in registers or spilled, across the tile loop.
  auto fresh_lane = []() -> int {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
  };
  int n = walk.next(lane);
  if (n < 0) {
    // no active tile: O = 0, LSE = -FLT_MAX
    const int eln = fresh_lane();
    const int etq = m * kTile + wave * 32 + (eln & 31);
    const int ehd = eln >> 5;
    if (etq >= lq) return;
    uint16_t* op = p.out + ((int64_t)(t0 + etq) * p.Hq + h) * kHeadDim;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) *reinterpret_cast<v2i*>(op + d * 32 + 8 * r4 + 4 * ehd) = v2i{0, 0};
    if (p.lse != nullptr && ehd == 0) p.lse[(int64_t)h * p.T + t0 + etq] = kNegFltMax;
    return;
  }
  int n1 = walk.next(lane);
  int n2 = n1 >= 0 ? walk.next(lane) : -1;
  Pages pg_n = lookup(n, lane);
  Pages pg_1 = n1 >= 0 ? lookup(n1, lane) : Pages{0};
  Pages pg_2 = n2 >= 0 ? lookup(n2, lane) : Pages{0};
  pg_n.kv = __builtin_amdgcn_readfirstlane(pg_n.kv);
  pg_1.kv = __builtin_amdgcn_readfirstlane(pg_1.kv);
  pg_2.kv = __builtin_amdgcn_readfirstlane(pg_2.kv);

  // Prologue: K(n) and its descales; S(n), its scale, mask and maximum; then
  // K(n1) into the product tile.
  uint8_t* kslot0 = QK8 ? kmat_lds : kst_lds;  // where K(n) lands
  dma_tile(p.kc, n, pg_n.kv, kslot0, lane);
  dma_kscale(n, pg_n.kv, lane, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) widen_k(j, lane);
  __syncthreads();
  v16f sa[4], sb[4];
  {
    widen_q();
    qk_tile(sa, lane, QK8 ? k_offsets(lane) : v4i{}, kslot0);
    float tm = -INFINITY;
#pragma unroll
    for (int c = 0; c < 4; ++c) tm = prep_block(sa[c], ks_read(c, lane, 0), c, n, lane, tm);
    update_max(tm);
  }
  __syncthreads();  // every wave is done with K(n) and the descales of n
  if (n1 >= 0) {
    dma_tile(p.kc, n1, pg_1.kv, QK8 ? kmat_lds + kTile * kHeadDim : kst_lds, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) widen_k(j, lane);
    __syncthreads();
  }

  // One step: S(n) in `cur`, S(n1) into `nxt`.  FP8 products: K(n1) is in
  // ring slot `par`, and K(n2) goes to slot par^1, which held K(n).
  auto step = [&](v16f* cur, v16f* nxt, auto par_tag) {
    constexpr int par = decltype(par_tag)::value;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    int tl = tid;  // (opaque, like ln: the offsets are loaded, not derived)
    if constexpr (QK8) asm volatile("" : "+v"(tl));
    // The first K operands of phase A (from the ring slot that already holds
    // K(n1)) are read before anything else, so that their LDS round trip,
    // and the offset table's before it, pass behind the tile walk and the
    // loads below.  K operands are read kAhead products ahead, through the
    // block boundaries.
    const uint8_t* k1 = QK8 ? kmat_lds + par * kTile * kHeadDim : kmat_lds;
    const v4i ko = QK8 ? *reinterpret_cast<const v4i*>(&ofs_lds[tl * 8]) : v4i{};
    constexpr int kRing = kAhead + 1;
    KOp ring[kRing];
#pragma unroll
    for (int j = 0; j < kAhead; ++j) ring[j] = kop(j, ln, ko, k1);
    // the next tile and its page ids (a mask-chunk load inside the walk is
    // waited for at once, which must not also wait for the tile loads)
    const int n3 = n2 >= 0 ? walk.next(ln) : -1;
    const Pages pg_3 = n3 >= 0 ? lookup(n3, ln) : Pages{0};
    // loads of the step: V(n), the descales of n1, K(n2); on the FP8 paths V
    // and the descales alternate between two buffers by step parity
    constexpr int vs = QK8 ? par : 0;
    dma_tile(p.vc, n, pg_n.kv, v8_lds + vs * kTile * kHeadDim, ln);
    if (n1 >= 0) dma_kscale(n1, pg_1.kv, ln, vs);
    uint8_t* k2dst = QK8 ? kmat_lds + (par ^ 1) * kTile * kHeadDim : kst_lds;
    if (n2 >= 0) dma_tile(p.kc, n2, pg_2.kv, k2dst, ln);

    // ---- A: exponentials of S(n), products of S(n1) ------------------------
    v8i pk[2];
    float ls = 0.0f;
    // Block by block, so that S(n) frees its registers as S(n1) needs them;
    // the K operands of block c+1 are read while block c computes, and the
    // E4M3 codes and partial sum of each block are pinned in this phase (the
    // compiler would otherwise sink the whole softmax to P.V, past the
    // barrier).  The products run even after the last tile, on whatever the
    // K tile holds, and are not used: an assignment on one path only would
    // keep the old contents of `nxt` alive through the whole phase.
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v16f acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < kPerBlock; ++ks) {
        const int j = c * kPerBlock + ks;
        if (j + kAhead < 4 * kPerBlock) ring[(j + kAhead) % kRing] = kop(j + kAhead, ln, ko, k1);
        acc = mfma_qk(ring[j % kRing], ks, acc);
      }
      nxt[c] = acc;
      ls += exp_block(cur[c], c, pk);
      asm volatile("" : "+v"(pk[c >> 1]), "+v"(ls));
      // interleave: each product with its operand read and a share of the softmax
#pragma unroll
      for (int ks = 0; ks < kPerBlock; ++ks) {
        if constexpr (SPLIT) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
          __builtin_amdgcn_sched_group_barrier(0x002, 12, 0); // VALU
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 12, 0); // VALU
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, QK8 ? 2 : 1, 0);      // DS read
          __builtin_amdgcn_sched_group_barrier(0x002, QK8 ? 24 : 6, 0);     // VALU
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run = l_run * (rescale ? alpha : 1.0f) + ls;

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // K(n1) no longer read; V(n), descales of n1 and K(n2) are in LDS

    // ---- B: O *= alpha, O += V(n) P(n); maximum of S(n1); widen K(n2) -------
    // Per 32-dim output block d: its two products (operands read one block
    // ahead), then, while they run, a quarter of the widening of K(n2), the
    // scale, mask and maximum of block d of S(n1), and the next block's V
    // operands and rescale.  The widening also runs after the last tiles, on
    // stale data that no product reads.
    // (the factor is exactly 1 when no row of the wave has a new maximum;
    // multiplying anyway keeps the phase free of branches)
    const float sc = rescale ? alpha : 1.0f;
    const v4i vo = QK8 ? *reinterpret_cast<const v4i*>(&ofs_lds[tl * 8 + 4]) : v4i{};
    v8i va0 = vread(0, ln, vo, vs), va1 = vread(4, ln, vo, vs);
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[0][r] *= sc;
    float tm = -INFINITY;
    // A band tile of S(n1) gets its descales and mask for all four blocks
    // here, and the block loop below then scales it by the descale slot of
    // 1.0: the loop has no branch, so the scheduler can move the next block's
    // operand reads ahead of the current block's maximum.
    const bool band1 = band_tile(n1);
    if (band1) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        scale_block(nxt[d], ks_read(d, ln, vs));
        mask_block(nxt[d], d, n1, ln);
      }
    }
    const int kslot = band1 ? kOnes : vs;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      oacc[d] = mfma_f8(va0, pk[0], oacc[d]);
      oacc[d] = mfma_f8(va1, pk[1], oacc[d]);
      {
        const v16f kd = ks_read(d, ln, kslot);  // dead before the next block's V operands are read
        widen_k(d, ln);
        scale_block(nxt[d], kd);
        tm = max_block(nxt[d], tm);
      }
      if (d < 3) {
        va0 = vread(d + 1, ln, vo, vs);
        va1 = vread(5 + d, ln, vo, vs);
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d + 1][r] *= sc;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (n1 >= 0) update_max(tm);
    // f16 path: V(n) and the descales are no longer read, and K(n2) is
    // widened.  The FP8 paths need no barrier here: the next step writes the
    // other V and descale buffers and the K slot that held K(n1), and no wave
    // starts it before every wave has passed this step's barrier, i.e. is done
    // with the products that read K(n1) and with the previous step's P.V.
    if constexpr (!QK8) __syncthreads();
    n = n1;
    n1 = n2;
    n2 = n3;
    pg_n = pg_1;
    pg_1 = pg_2;
    pg_2 = pg_3;
    // the K/V page id is wave-uniform and its load has completed (it was
    // waited for before the barrier): keep it in a scalar register
    pg_2.kv = __builtin_amdgcn_readfirstlane(pg_2.kv);
  };
  while (true) {
    step(sa, sb, std::integral_constant<int, 1>{});
    if (n < 0) break;
    step(sb, sa, std::integral_constant<int, 0>{});
    if (n < 0) break;
  }

  // ---- epilogue ------------------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  // (the V descale is read here too rather than kept live across the loop)
  const int eln = fresh_lane();
  const int etq = m * kTile + wave * 32 + (eln & 31);
  const int ehd = eln >> 5;
  if (etq >= lq) return;
  const bool empty = !(l_tot > 0.0f);
  const float vdesc = QUANT == BSA_QUANT_Q_TOKHEAD_K_TENSOR_V_TENSOR ? p.vscale[0] : p.vscale[g];
  const float inv = empty ? 0.0f : vdesc / l_tot;
  uint16_t* op = p.out + ((int64_t)(t0 + etq) * p.Hq + h) * kHeadDim;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = d * 32 + 8 * r4 + 4 * ehd;
      const uint32_t w0 = (uint32_t)f32_to_bf16_rne(oacc[d][4 * r4 + 0] * inv) |
                          ((uint32_t)f32_to_bf16_rne(oacc[d][4 * r4 + 1] * inv) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16_rne(oacc[d][4 * r4 + 2] * inv) |
                          ((uint32_t)f32_to_bf16_rne(oacc[d][4 * r4 + 3] * inv) << 16);
      *reinterpret_cast<v2i*>(op + d0) = v2i{(int)w0, (int)w1};
    }
  }
  if (p.lse != nullptr && ehd == 0) {
    p.lse[(int64_t)h * p.T + t0 + etq] = empty ? kNegFltMax : (m_run + log2f(l_tot) - p.pscale_log2) * kLn2;
  }
}

}  // namespace

extern "C" {

int bsa_fp8_prefill_ex(const void* q, const void* kcache, const void* vcache, const float* qscale,
                       const float* kscale, const float* vscale, const int32_t* cu_seqlens_q,
                       const int32_t* block_table, const int32_t* seqlens_kv, const uint8_t* block_mask,
                       int quant_type, int page_size, const bsa_fp8_dims* dims,
                       const bsa_fp8_options* options, void* out, float* lse, void* stream) {
  // ---- static validation (host only, before any HIP call) ----
  bsa::Resolved r;
  const int st = bsa::resolve(dims, block_mask, options, &r);
  if (st != BSA_OK) return st;
  if (page_size != 32 && page_size != 64) return BSA_ERR_PAGE_SIZE;
  if (quant_type != BSA_QUANT_Q_TOKHEAD_K_TENSOR_V_TENSOR &&
      quant_type != BSA_QUANT_Q_TOKHEAD_K_TOKHEAD_V_HEAD)
    return BSA_ERR_QUANT_TYPE;
  const bsa_fp8_dims& d = r.d;
  const int64_t grid = r.tasks;
  if (grid > 0) {
    if (q == nullptr || kcache == nullptr || vcache == nullptr || qscale == nullptr ||
        kscale == nullptr || vscale == nullptr || cu_seqlens_q == nullptr ||
        block_table == nullptr || seqlens_kv == nullptr || out == nullptr)
      return BSA_ERR_NULL_POINTER;
  }
  if (grid == 0) return BSA_OK;

  Params p;
  p.q = static_cast<const uint8_t*>(q);
  p.kc = static_cast<const uint8_t*>(kcache);
  p.vc = static_cast<const uint8_t*>(vcache);
  p.qscale = qscale;
  p.kscale = kscale;
  p.vscale = vscale;
  p.cu_q = cu_seqlens_q;
  p.block_table = block_table;
  p.seqlens_kv = seqlens_kv;
  p.mask = block_mask;
  p.sidx = r.sidx;
  p.slen = r.slen;
  p.schedule = r.schedule;
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.B = d.batch;
  p.T = d.total_q;
  p.Hq = d.num_heads_q;
  p.Hkv = d.num_heads_kv;
  p.group = r.group;
  p.page_size = page_size;
  p.page_shift = page_size == 64 ? 6 : 5;
  p.max_pages = d.max_pages_per_seq;
  p.mt = d.mask_tiles_q;
  p.mkv = d.mask_tiles_kv;
  p.mt_grid = r.mt_grid;
  p.layout = d.kv_layout;
  p.causal = d.causal;
  p.qk_scale = d.softmax_scale * kLog2e;
  p.pscale_log2 = log2f(r.p_scale);
  p.q_tok_stride = r.q_layout == BSA_Q_TND ? d.num_heads_q : 1;
  p.q_head_stride = r.q_layout == BSA_Q_TND ? 1 : d.total_q;
  p.page_bytes = (uint32_t)page_size * (uint32_t)d.num_heads_kv * kHeadDim;
  p.slot_stride = d.kv_layout == BSA_KV_NHD ? d.num_heads_kv : 1;
  p.head_stride = d.kv_layout == BSA_KV_NHD ? 1 : page_size;

  const dim3 grid3((unsigned)grid), block3(kThreads);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool list = r.form == bsa::kFormList;
  const bool q1 = quant_type == BSA_QUANT_Q_TOKHEAD_K_TOKHEAD_V_HEAD;
  constexpr int Q0 = BSA_QUANT_Q_TOKHEAD_K_TENSOR_V_TENSOR, Q1 = BSA_QUANT_Q_TOKHEAD_K_TOKHEAD_V_HEAD;
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid3, block3, 0, s, p); };
  auto pick = [&](auto qkm) {
    constexpr int M = decltype(qkm)::value;
    if (q1) list ? go(bsa_fp8_prefill_kernel<Q1, kFormList, M>) : go(bsa_fp8_prefill_kernel<Q1, 0, M>);
    else list ? go(bsa_fp8_prefill_kernel<Q0, kFormList, M>) : go(bsa_fp8_prefill_kernel<Q0, 0, M>);
  };
  if (r.qk == BSA_QK_FP8) pick(std::integral_constant<int, kQkFp8>{});
  else if (r.qk == BSA_QK_FP8_SPLIT) pick(std::integral_constant<int, kQkFp8Split>{});
  else pick(std::integral_constant<int, kQkF16>{});
  if (hipGetLastError() != hipSuccess) return BSA_ERR_LAUNCH;
  return BSA_OK;
}

int bsa_fp8_prefill(const void* q, const void* kcache, const void* vcache, const float* qscale,
                    const float* kscale, const float* vscale, const int32_t* cu_seqlens_q,
                    const int32_t* block_table, const int32_t* seqlens_kv, const uint8_t* block_mask,
                    int quant_type, int page_size, const bsa_fp8_dims* dims, void* out, float* lse,
                    void* stream) {
  return bsa_fp8_prefill_ex(q, kcache, vcache, qscale, kscale, vscale, cu_seqlens_q, block_table,
                            seqlens_kv, block_mask, quant_type, page_size, dims, nullptr, out, lse,
                            stream);
}

}  // extern "C"
