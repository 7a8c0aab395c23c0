// Block-sparse FP8 (E4M3) attention prefill over a paged KV cache, gfx950.
//
// One workgroup of 256 threads (4 waves) owns one (sequence, q-head, 128-query
// tile); wave w owns queries 32w..32w+31.  Two workgroups share a CU so that
// one's softmax (VALU) overlaps the other's matrix products.
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
//   2. Per active tile, K and V rows are gathered from the paged cache (one
//      page-table lookup per row).  V (and, for per-token K scales, the K
//      descales) go straight to LDS with direct-to-LDS loads, double-buffered;
//      K goes through registers, one tile ahead.
//   3. S^T = K . Q^T.  E4M3 -> f16 is exact (a bit shift that scales values by
//      2^-8), so K is widened to f16 once per workgroup when it is staged in
//      LDS and Q once in registers, and the product runs on
//      v_mfma_f32_32x32x16_f16, whose accumulation is fp32-accurate.  (The
//      E4M3 matrix path keeps only about 14 bits below the largest product of
//      a dot product, which moves P across E4M3 rounding boundaries.)
//      Computing S^T makes every lane own one query, so the running max, sum
//      and rescale are per lane.  K rows are read in a permuted order so that
//      the accumulator registers of lane half h hold keys h*32..h*32+31 of each
//      64-key half of the tile, in register order.
//   4. Online softmax in fp32 in the log2 domain: qscale*softmax_scale*log2(e)
//      (and the per-tensor K descale, and 2^16 for the f16 widening) is one
//      per-lane constant; P' = exp2(x - m + log2(p_scale)) = p_scale*exp(score
//      - max), so the P-scale (256 by default: hpc-ops article, "FP8 Tensor
//      Core compute: fixed P-scale quantisation"; any p_scale in (0, 448]:
//      "Quant Block Sparse Attention", "Key parameters") costs nothing.  P' is
//      rounded to E4M3
//      (v_cvt_pk_fp8_f32, round to nearest even) and the row sum keeps the
//      unrounded P'.  The accumulator rescale is skipped when no row of the
//      wave has a new maximum (the factor is then exactly 1).
//   5. O^T += V^T . P^T on v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3).  V stays
//      row-major in LDS; the transposing read ds_read_b64_tr_b8 delivers it
//      key-major.
//   6. Epilogue: O = O_acc * vdescale / sum(P') (the 1/p_scale is inside the
//      sum), written as bf16; LSE = ln2 * (m + log2(sum) - log2(p_scale)).  A query whose sparse
//      set is empty gets O = 0 and LSE = -FLT_MAX ("Quant Block Sparse
//      Attention", "Sparse indices & PA page table").

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

// 16-byte chunk swizzle of the fp8 V rows (128 B, 8 chunks) in LDS.
__device__ __forceinline__ int swz8(int row) { return (row & 7) ^ (((row >> 5) & 1) << 2); }


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

template <int QUANT, int FORM, bool QK8>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
bsa_fp8_prefill_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) uint8_t k16_lds[kTile * kK16Row];       // 32 KB
  __shared__ __attribute__((aligned(16))) uint8_t v8_lds[2][kTile * kHeadDim];    // 32 KB
  __shared__ __attribute__((aligned(16))) float ks_lds[2][kTile];                 // 1 KB

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hd = lane >> 5;   // lane half
  const int col = lane & 31;  // query column owned by this lane within the wave

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

  // Q operand (B of S^T = K.Q^T, f16 32x32x16): lane holds query `col`,
  // head-dim elements ks*16 + hd*8 .. +7 for ks = 0..7.
  v8h qh[8];
  v8i q8[2];  // FP8 products: lane holds query `col`, dims ks*64 + hd*32 .. +31
  float cscale = 0.0f;
  if constexpr (QK8) {
    if (q_valid) {
      const int64_t qi = (int64_t)(t0 + tq) * p.q_tok_stride + (int64_t)h * p.q_head_stride;
      const uint8_t* qp = p.q + qi * kHeadDim + hd * 32;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) q8[ks] = *reinterpret_cast<const v8i*>(qp + ks * 64);
      cscale = p.qscale[qi] * p.qk_scale;
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) q8[ks] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    }
  } else {
    v2i raw[8];
    if (q_valid) {
      const int64_t qi = (int64_t)(t0 + tq) * p.q_tok_stride + (int64_t)h * p.q_head_stride;
      const uint8_t* qp = p.q + qi * kHeadDim + hd * 8;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) raw[ks] = *reinterpret_cast<const v2i*>(qp + ks * 16);
      cscale = p.qscale[qi] * p.qk_scale;
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) raw[ks] = v2i{0, 0};
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const v2i a = e4m3x4_to_f16x4((uint32_t)raw[ks][0]);
      const v2i c = e4m3x4_to_f16x4((uint32_t)raw[ks][1]);
      const v4i w = v4i{a[0], a[1], c[0], c[1]};
      qh[ks] = __builtin_bit_cast(v8h, w);
    }
  }
  if (QUANT == BSA_QUANT_Q_TOKHEAD_K_TENSOR_V_TENSOR) cscale *= p.kscale[0];
  // Keep the score constant strictly positive so that a masked score (-inf)
  // maps to exp2(-inf) = 0 without a select.  With descales >= 0 this only
  // changes a zero constant, where every x is then ~1e-38 * S instead of 0.
  cscale = fmaxf(cscale, 1.17549435e-38f);
  const float vdesc = QUANT == BSA_QUANT_Q_TOKHEAD_K_TENSOR_V_TENSOR ? p.vscale[0] : p.vscale[g];

  v16f oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[d][r] = 0.0f;
  float m_run = -INFINITY;  // running max of x = score * log2(e)
  float l_run = 0.0f;       // this lane's half of sum(P'), P' = 2^(x - m + 8)

  // K operand rows: accumulator row i of block c holds key
  // (c>>1)*64 + hi*32 + (c&1)*16 + ri with hi = (i>>2)&1, ri = (i>>3)*4 + (i&3).

  // Staging roles: K through registers, one row per thread (row tid & 127,
  // head-dim bytes 64*(tid>>7) .. +63); V by direct-to-LDS loads (wave w: rows
  // 32w..32w+31, 8 rows of 128 bytes per instruction).
  const int32_t* bt = p.block_table + (int64_t)b * p.max_pages;
  const int khalf = wave >> 1;
  v4i kreg[4];

  // Loads of a tile come in three parts, spread over iterations so that no
  // memory latency sits on the critical path:
  //  * lookup(n): the page-table entries of tile n, issued two tiles ahead and
  //    waited only at the top of the next iteration (the VMEM counter drains
  //    in order, so a lookup waited right before the data loads that need it
  //    would expose a full memory round trip every tile);
  //  * issue_k(n): the K rows of tile n into registers, one tile ahead;
  //  * issue_v(n): the V rows (and per-token K descales) of tile n straight
  //    into LDS, issued after the current tile's PV so that no direct-to-LDS
  //    load is in flight while LDS operands are read (the compiler can then
  //    wait for exact LDS counts).
  // Rows past the KV length are redirected to row lkv-1 (valid; every lookup
  // index is at most (lkv-1)/page_size): their K is zeroed and their P is 0.
  // The 32 V rows of a wave lie in one 32-aligned block, hence in one page.
  struct PageSet {
    int k, v, ks;
  };
  // (vzero keeps the V page lookup a per-lane load: a wave-uniform one is moved
  // to a scalar register at once, which waits for every load in flight)
  int vzero = 0;
  asm volatile("" : "+v"(vzero));
  // K row staged by this thread: (wave & 1) * 64 + lane.
  auto lookup = [&](int n, int ln) -> PageSet {
    PageSet ps;
    ps.k = bt[min(n * kTile + (wave & 1) * 64 + ln, lkv - 1) >> p.page_shift];
    ps.v = bt[min(n * kTile + wave * 32 + vzero, lkv - 1) >> p.page_shift];
    ps.ks = QUANT == BSA_QUANT_Q_TOKHEAD_K_TOKHEAD_V_HEAD
                ? bt[min(n * kTile + (wave & 1) * 64 + ln, lkv - 1) >> p.page_shift]
                : 0;
    return ps;
  };
  // Byte offset of (page, slot, this kv-head) in a cache: one 32x32->64-bit
  // product per page plus 32-bit in-page arithmetic.
  const int head_row = g * p.head_stride;
  auto row_addr = [&](const uint8_t* base, int pg, int slot) -> const uint8_t* {
    return base + (uint64_t)(uint32_t)pg * p.page_bytes + (uint32_t)(slot * p.slot_stride + head_row) * kHeadDim;
  };
  const int pmask = p.page_size - 1;
  // (rows past the KV length are zeroed when K is widened, not here: a select
  // on the loaded registers would make the loads complete at once)
  auto issue_k = [&](int n, const PageSet& ps, int ln) {
    const int slot = min(n * kTile + (wave & 1) * 64 + ln, lkv - 1) & pmask;
    const v4i* src = reinterpret_cast<const v4i*>(row_addr(p.kc, ps.k, slot) + khalf * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) kreg[i] = src[i];
  };
  auto issue_v = [&](int n, int buf, const PageSet& ps, int ln) {
    const int row0 = wave * 32 + (ln >> 3);
    if (n * kTile + kTile <= lkv) {
      // Whole tile inside the KV length: the wave's 32 rows are consecutive
      // slots of one page.
      const uint8_t* src0 = row_addr(p.vc, ps.v, (n * kTile + row0) & pmask);
      const uint32_t step = 8u * (uint32_t)p.slot_stride * kHeadDim;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds((glb_void*)(src0 + i * step + (((ln & 7) ^ swz8(row0 + i * 8)) << 4)),
                                         (lds_void*)(&v8_lds[buf][(wave * 32 + i * 8) * kHeadDim]), 16, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = row0 + i * 8;
        const int j = min(n * kTile + row, lkv - 1);
        const uint8_t* src = row_addr(p.vc, ps.v, j & pmask) + (((ln & 7) ^ swz8(row)) << 4);
        __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)(&v8_lds[buf][(wave * 32 + i * 8) * kHeadDim]), 16, 0, 0);
      }
    }
    if (QUANT == BSA_QUANT_Q_TOKHEAD_K_TOKHEAD_V_HEAD && wave < 2) {
      const int slot = min(n * kTile + wave * 64 + ln, lkv - 1) & pmask;
      const float* src = p.kscale + (uint64_t)(uint32_t)ps.ks * (p.page_bytes / kHeadDim) + (uint32_t)(slot * p.slot_stride + head_row);
      __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)(&ks_lds[buf][wave * 64]), 4, 0, 0);
    }
  };

  // n: tile being processed (LDS buffer parity `buf` of the step); n1: the
  // next one.  Page ids live in pg[parity of the tile's position], so no copy
  // of a pending load result is ever needed.
  int n = walk.next(lane);
  int n1 = -1;
  PageSet pg[2] = {{0, 0, 0}, {0, 0, 0}};
  if (n >= 0) {
    pg[0] = lookup(n, lane);
    issue_k(n, pg[0], lane);
    issue_v(n, 0, pg[0], lane);
    n1 = walk.next(lane);
    if (n1 >= 0) pg[1] = lookup(n1, lane);
  }

  // One active tile; BUF is the LDS buffer holding its V (and K descales).
  auto tile_step = [&](auto buf_tag) {
    constexpr int buf = decltype(buf_tag)::value;
    // Lane-derived offsets are recomputed from an opaque copy of the lane id
    // every tile instead of being held in registers across the loop.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lhd = ln >> 5;
    const int lcol = ln & 31;
    const int krow = (wave & 1) * 64 + ln;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // k16 and the other V buffer are no longer read; this tile's V is in LDS
    // Widen this tile's K to f16 in LDS.  Layout is chunk-major: the 16-byte
    // chunk c (head-dim elements 8c..8c+7) of key row r sits at c*2048 + r*16.
    if (n * kTile + krow >= lkv) {
#pragma unroll
      for (int i = 0; i < 4; ++i) kreg[i] = v4i{0, 0, 0, 0};
    }
    if constexpr (QK8) {
      // E4M3 kept as is, chunk-major: 16-byte chunk c (dims 16c..16c+15) of
      // key row r at c*2048 + r*16.
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<v4i*>(k16_lds + (4 * khalf + i) * 2048 + krow * 16) = kreg[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v2i a = e4m3x4_to_f16x4((uint32_t)kreg[i][0]);
        const v2i c = e4m3x4_to_f16x4((uint32_t)kreg[i][1]);
        const v2i d = e4m3x4_to_f16x4((uint32_t)kreg[i][2]);
        const v2i e = e4m3x4_to_f16x4((uint32_t)kreg[i][3]);
        const int chunk = 8 * khalf + 2 * i;
        *reinterpret_cast<v4i*>(k16_lds + chunk * 2048 + krow * 16) = v4i{a[0], a[1], c[0], c[1]};
        *reinterpret_cast<v4i*>(k16_lds + (chunk + 1) * 2048 + krow * 16) = v4i{d[0], d[1], e[0], e[1]};
      }
    }
    __syncthreads();  // k16 ready
    if (n1 >= 0) issue_k(n1, pg[buf ^ 1], ln);
    const int n2 = n1 >= 0 ? walk.next(ln) : -1;
    if (n2 >= 0) pg[buf] = lookup(n2, ln);

    // ---- S^T = K . Q^T (f16 operands, fp32 accumulation) ------------------
    // k-step outer, 32-key block inner: four independent accumulation chains,
    // and the operands of step ks+1 are read from LDS before the products of
    // step ks are issued, so LDS latency hides behind the matrix pipe.
    v16f s[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[c][r] = 0.0f;
    if constexpr (QK8) {
      // FP8 products (v_mfma_f32_32x32x64_f8f6f4): two k-steps of 64 dims;
      // lane half h reads dims ks*64 + 32h .. +31 of its key row (chunks
      // 4ks + 2h and 4ks + 2h + 1).
      const int hi_a = (lcol >> 2) & 1;
      const int ri_a = ((lcol >> 3) << 2) | (lcol & 3);
      const uint8_t* kp = k16_lds + 2 * lhd * 2048 + (hi_a * 32 + ri_a) * 16;
      auto kread = [&](int c, int ks) -> v8i {
        const uint8_t* a = kp + ((c >> 1) * 64 + (c & 1) * 16) * 16 + ks * 4 * 2048;
        const v4i lo = *reinterpret_cast<const v4i*>(a);
        const v4i hi = *reinterpret_cast<const v4i*>(a + 2048);
        return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      };
      v8i ka[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) ka[x] = kread(x & 3, x >> 2);
#pragma unroll
      for (int x = 0; x < 8; ++x) s[x & 3] = mfma_f8(ka[x], q8[x >> 2], s[x & 3]);
    } else {
      const int hi_a = (lcol >> 2) & 1;
      const int ri_a = ((lcol >> 3) << 2) | (lcol & 3);
      const uint8_t* kp = k16_lds + lhd * 2048 + (hi_a * 32 + ri_a) * 16;
      auto kaddr = [&](int c, int ks) { return kp + ((c >> 1) * 64 + (c & 1) * 16) * 16 + ks * 4096; };
      v8h acur[4], anxt[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) acur[c] = *reinterpret_cast<const v8h*>(kaddr(c, 0));
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        if (ks < 7) {
#pragma unroll
          for (int c = 0; c < 4; ++c) anxt[c] = *reinterpret_cast<const v8h*>(kaddr(c, ks + 1));
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) s[c] = mfma_f16(acur[c], qh[ks], s[c]);
#pragma unroll
        for (int c = 0; c < 4; ++c) acur[c] = anxt[c];
      }
      // Keep four operand reads in flight ahead of the matrix products.
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);    // DS read
#pragma unroll
      for (int k = 0; k < 14; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    __builtin_amdgcn_sched_barrier(0);

    // Lane holds, for its query, keys key(c, r) = (c>>1)*64 + hd*32 + (c&1)*16 + r.
    if (QUANT == BSA_QUANT_Q_TOKHEAD_K_TOKHEAD_V_HEAD) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float* ksp = &ks_lds[buf][(c >> 1) * 64 + lhd * 32 + (c & 1) * 16];
#pragma unroll
        for (int r = 0; r < 16; ++r) s[c][r] *= ksp[r];
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const bool band = (p.causal && n * kTile + kTile - 1 > p_wave_min) || (n * kTile + kTile > lkv);
    if (band) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = n * kTile + (c >> 1) * 64 + lhd * 32 + (c & 1) * 16 + r;
          const bool ok = j < lkv && (!p.causal || j <= p_wave_min + lcol);
          s[c][r] = ok ? s[c][r] : -INFINITY;
        }
    }

    // ---- online softmax ------------------------------------------------------
    // row max as a tree (eight independent partial maxima)
    float pm[8];
#pragma unroll
    for (int q8 = 0; q8 < 8; ++q8) {
      const int c = q8 >> 1, r0 = (q8 & 1) * 8;
      pm[q8] = max3f(max3f(s[c][r0], s[c][r0 + 1], s[c][r0 + 2]), max3f(s[c][r0 + 3], s[c][r0 + 4], s[c][r0 + 5]),
                     fmaxf(s[c][r0 + 6], s[c][r0 + 7]));
    }
    float tmax = fmaxf(max3f(pm[0], pm[1], pm[2]), max3f(pm[3], pm[4], max3f(pm[5], pm[6], pm[7])));
    {
      // other lane half (keys of the other 32-row halves): v_permlane32_swap
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float tmax_x = tmax == -INFINITY ? -INFINITY : tmax * cscale;
    const float m_new = fmaxf(m_run, tmax_x);
    const float m_safe = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_safe);  // exp2(-inf) = 0
    const float bias = p.pscale_log2 - m_safe;
    const bool rescale = __ballot(m_new != m_run) != 0;
    m_run = m_new;

    v8i pk[2];
    float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        // masked scores are -inf and cscale > 0, so their P' is exactly 0
        const float e0 = __builtin_amdgcn_exp2f(fmaf(s[c][r], cscale, bias));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(s[c][r + 1], cscale, bias));
        const float e2 = __builtin_amdgcn_exp2f(fmaf(s[c][r + 2], cscale, bias));
        const float e3 = __builtin_amdgcn_exp2f(fmaf(s[c][r + 3], cscale, bias));
        ls[r >> 2] += (e0 + e1) + (e2 + e3);
        // bytes (c&1)*16 + r .. +3 of the P operand of PV step c>>1
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, w, true);
        pk[c >> 1][(c & 1) * 4 + (r >> 2)] = w;
      }
    }
    if (rescale) {
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
    }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);

    // ---- O^T += V^T . P^T ----------------------------------------------------
    // Transposing read: in each 16-lane group, source lane 2k+q addresses key
    // row (step*64 + half*32 + 8*rr + k) at head-dim column base + 8q; result
    // lane i then holds column base + i for those 8 keys.
    // Rows sp*64 + half*32 + 8*rr + kk all share this lane's chunk swizzle, so
    // one base per head-dim block d serves the whole tile.
    const int grp = ln >> 4;
    const int kk = (ln & 15) >> 1;
    const int half = grp >> 1;
    const int csw = (grp & 1) ^ kk ^ (half << 2);  // logical chunk 2d + (grp&1), swizzled
    const uint8_t* vrow0 = v8_lds[buf] + (half * 32 + kk) * kHeadDim + 8 * (ln & 1);
    auto vread = [&](int x) -> v8i {  // x = sp*4 + d
      const uint8_t* vp = vrow0 + (((2 * (x & 3)) ^ csw) << 4) + (x >> 2) * 64 * kHeadDim;
      v8i a;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vp + rr * 8 * kHeadDim));
        a[2 * rr] = t[0];
        a[2 * rr + 1] = t[1];
      }
      return a;
    };
    {
      // operands of the next product are read while the current one runs
      v8i va[8];
      va[0] = vread(0);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        if (x + 1 < 8) va[x + 1] = vread(x + 1);
        oacc[x & 3] = mfma_f8(va[x], pk[x >> 2], oacc[x & 3]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);    // DS read
#pragma unroll
      for (int k = 0; k < 7; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    if (n1 >= 0) issue_v(n1, buf ^ 1, pg[buf ^ 1], ln);
    n = n1;
    n1 = n2;
  };
  while (n >= 0) {
    tile_step(std::integral_constant<int, 0>{});
    if (n < 0) break;
    tile_step(std::integral_constant<int, 1>{});
  }

  // ---- epilogue ------------------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!q_valid) return;
  const bool empty = !(l_tot > 0.0f);
  const float inv = empty ? 0.0f : vdesc / l_tot;
  uint16_t* op = p.out + ((int64_t)(t0 + tq) * p.Hq + h) * kHeadDim;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = d * 32 + 8 * r4 + 4 * hd;
      const uint32_t w0 = (uint32_t)f32_to_bf16_rne(oacc[d][4 * r4 + 0] * inv) |
                          ((uint32_t)f32_to_bf16_rne(oacc[d][4 * r4 + 1] * inv) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16_rne(oacc[d][4 * r4 + 2] * inv) |
                          ((uint32_t)f32_to_bf16_rne(oacc[d][4 * r4 + 3] * inv) << 16);
      *reinterpret_cast<v2i*>(op + d0) = v2i{(int)w0, (int)w1};
    }
  }
  if (p.lse != nullptr && hd == 0) {
    p.lse[(int64_t)h * p.T + t0 + tq] = empty ? kNegFltMax : (m_run + log2f(l_tot) - p.pscale_log2) * kLn2;
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
  if (r.qk8) {
    if (q1) list ? go(bsa_fp8_prefill_kernel<Q1, kFormList, true>) : go(bsa_fp8_prefill_kernel<Q1, 0, true>);
    else list ? go(bsa_fp8_prefill_kernel<Q0, kFormList, true>) : go(bsa_fp8_prefill_kernel<Q0, 0, true>);
  } else {
    if (q1) list ? go(bsa_fp8_prefill_kernel<Q1, kFormList, false>) : go(bsa_fp8_prefill_kernel<Q1, 0, false>);
    else list ? go(bsa_fp8_prefill_kernel<Q0, kFormList, false>) : go(bsa_fp8_prefill_kernel<Q0, 0, false>);
  }
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
