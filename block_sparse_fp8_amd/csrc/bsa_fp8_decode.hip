// FP8 sparse decode over a paged cache of 656-byte token rows, gfx950.
//
// The workload of the FlashMLA FP8 sparse decoding article: multi-query
// attention (every query head reads the same single KV head) with 576-dim keys
// (512 E4M3 values in four 1x128 tiles with one float32 descale each, then 64
// bfloat16 values) and 512-dim values (the first 512 key dimensions); each
// query token attends to its own list of top-k cache rows, each named as
// page-block index * page_block_size + offset in the block, -1 for an unused
// entry (the article's quick-reproduce paragraph).  The article's
// kernel dequantises K/V to bfloat16 and runs both products on bfloat16 matrix
// units; the same split holds here.  Its two thread blocks per query token
// each dequantise half of the rows and exchange them; here one workgroup
// serves all heads of a query token (up to 128, 16 per wave), so every row is
// read and dequantised once.
//
// Per workgroup (sequence b, query token s, 16*NW heads), the list is walked
// 32 tokens ("a block") at a time, one step per block with one barrier at its
// end; every global load inside the loop is a direct-to-LDS load, so each wait
// is an exact count of them.  Step n:
//   row ids: every wave copies the 32 entries of block n+3 into a ring of six
//      blocks in LDS (an entry is used only if it lies in the list and names a
//      row: 0 <= entry < num_pages * page_size).
//   S^T = K . Q^T of block n on v_mfma_f32_16x16x32_bf16, wave w owning heads
//      16w..16w+15; tokens sit in the K tile in the order those reads want, so
//      each lane holds 8 consecutive tokens of one head, the layout of the P
//      operand below.
//   dequantise block n+1: E4M3 -> fp32, times the tile's descale, -> bfloat16
//      (round to nearest even) into one of three bfloat16 K tiles [32
//      tokens][576] in LDS, plus the 64 bfloat16 values; each wave converts
//      its own tokens from its own staging region, and then refills that
//      region with the rows of block n+2 (41 chunks of 16 bytes per row, 16
//      lanes per row) without waiting for the other waves.
//   O^T += V^T . P^T of block n-1: wave w owns 512/NW output dims for all
//      heads, so each V value is read from LDS once per workgroup; V^T comes
//      from the row-major K tile through the transposing read
//      ds_read_b64_tr_b16.
//   online softmax of block n in the log2 domain with a lazily moved reference
//      maximum; P rounded to bfloat16 into one of two LDS buffers.
// A K tile is rewritten two steps after its Q.K^T and one after its P.V, a P
// buffer one step after its P.V, so the barrier at the end of each step orders
// every reuse.
// Epilogue: O = O_acc / l per head, bfloat16; LSE = ln sum exp(score).  A
// query with no valid index gets O = 0 and LSE = -FLT_MAX.
//
// Split lists (the article's launch grid also runs over "SM parts"): with
// num_splits > 1 the part index is the fastest-varying part of the workgroup
// id, part p walks only its own blocks of the list and stores O_p / l_p in
// fp32 and its log2-sum-exp in a caller workspace; a second kernel merges the
// parts of every (query token, head) by weights 2^(lse_p - max).

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <type_traits>

#include "bsa_fp8.h"
#include "bsa_internal.h"

#include <mutex>

namespace {

constexpr int kBlock = 32;          // tokens per iteration
constexpr int kDimK = 576;
constexpr int kDimV = 512;
constexpr int kRowBytes = 656;
constexpr int kKStride = kDimK * 2 + 32;   // bytes per LDS K row (padded: conflict-free reads)
constexpr int kMaxTopk = BSA_DECODE_MAX_TOPK;  // longest index list one workgroup walks (interface limit)
constexpr int kKTiles = 3;                 // K tiles: P.V of block n-1, Q.K^T of n, dequantisation of n+1
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegFltMax = -3.402823466e+38f;

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

struct DecodeParams {
  const uint16_t* q;          // bf16 [B, s_q, h_q, 576]
  const uint8_t* kv;          // [num_pages, page_size, 656]
  const int32_t* indices;     // [B, s_q, topk] cache rows (page * page_size + slot)
  uint16_t* out;              // bf16 [B, s_q, h_q, 512]
  float* lse;                 // [B, h_q, s_q] or nullptr
  int B, s_q, h_q, topk;
  int num_rows;               // num_pages * page_size: entries in [0, num_rows) name a row
  float score_scale;          // softmax_scale * log2(e)
  int num_splits;             // parts of each index list handled by separate workgroups
  int blocks_per_split;       // 32-token blocks per part
  float* opart;               // num_splits > 1: [splits, B*s_q, h_q, 512] normalised partial O
  float* lpart;               // num_splits > 1: [splits, B*s_q, h_q] partial log2-sum-exp (-inf: empty)
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a, b}, v2bf));
}

// Maximum / sum over lanes l, l^16, l^32, l^48 (the four lane groups holding
// one head's tokens), on the VALU: each swap returns this lane's value and its
// partner's.
__device__ __forceinline__ float max_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ v4f mfma_bf16(v4i a, v4i b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0,
                                                  0, 0);
}

// Direct-to-LDS load, 16 bytes per lane; a wave writes 64 consecutive chunks
// at the wave-uniform LDS address lds_addr.  Issued through asm so that the
// compiler does not make later LDS reads and barriers wait for it; every one
// is waited for explicitly.  M0 is set here and used by nothing else in this
// kernel.
__device__ __forceinline__ void dma_lds16(const void* gptr, uint32_t lds_addr) {
  // (the address is wave-uniform; readfirstlane keeps it in a scalar register
  // even where the compiler computed it with vector instructions)
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}
// Workgroup barrier that waits for this wave's LDS operations only.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Direct-to-LDS load of 4 bytes per active lane (lane l writes lds_addr + 4l).
__device__ __forceinline__ void dma_lds4(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gptr),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

// Staging of one block: for each group of 4 tokens ("set") a wave issues three
// rounds of 64 lanes x 16 bytes; lane (token tl = lane/16, part p = lane%16)
// of round 0 fetches codes 16p..16p+15 of its row, round 1 codes
// 256+16p..256+16p+15, round 2 the chunk 32+min(p, 8) (the four descales for
// p = 0, the bfloat16 values for p = 1..8; parts 9..15 repeat chunk 40).  So in
// each round a token's bytes are consecutive: codes 0..255 at 256*tl of round 0.
constexpr int kRound = 64 * 16;
constexpr int kRowRing = 6;        // blocks of row ids in LDS: n-1 .. n+5 around step n
// A head keeps its reference maximum until a block's maximum exceeds it by
// more than this (log2 units): P = 2^(x - reference) then stays below 2^8,
// which bfloat16 and the fp32 sums hold with the same relative rounding, and
// the accumulators are rescaled only when some head's reference moves.
constexpr float kLazyRescale = 8.0f;

// Row of token t (0..31) of a block in the LDS K tile.  The Q.K^T reads have
// lane c of each 16 read row c (tokens 8(c/4) + c%4) for the first product and
// row 16 + c (those tokens + 4) for the second, a pattern with no bank
// conflicts at a row stride of 1184 bytes.
__device__ __forceinline__ int krow(int t) { return ((t >> 2) & 1) * 16 + (t >> 3) * 4 + (t & 3); }

template <int NW>
__global__ void __launch_bounds__(NW * 64) bsa_fp8_decode_kernel(DecodeParams p) {
  constexpr int kHeads = 16 * NW;          // heads per workgroup
  constexpr int kDW = kDimV / NW;          // output dims per wave in P.V
  constexpr int kDB = kDW / 16;            // 16-dim blocks per wave
  constexpr int kSets = 8 / NW;            // groups of 4 tokens each wave stages and dequantises
  constexpr int kWaveStage = kSets * 3 * kRound;
  constexpr int kStageBytes = NW * kWaveStage;  // one block
  constexpr int kKTile = kBlock * kKStride;
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kKTiles * kKTile];
  __shared__ __attribute__((aligned(16))) uint8_t stage_lds[kStageBytes];  // one block, a region per wave
  __shared__ __attribute__((aligned(16))) uint8_t p_lds[2 * 4 * kHeads * 16];  // [block parity][token group][head][8 tokens]
  __shared__ __attribute__((aligned(16))) int32_t rows_lds[kRowRing * kBlock];
  __shared__ float alpha_lds[2 * kHeads];  // [block parity][head]
  __shared__ float l_lds[kHeads];
  __shared__ int rescale_lds[3];  // [block % 3]: some head's reference maximum moved

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 4;       // lane group
  const int c16 = lane & 15;     // column within a 16x16 block

  const int groups = p.h_q / kHeads;
  const int split = blockIdx.x % p.num_splits;
  const int rest = blockIdx.x / p.num_splits;
  const int hg = rest % groups;
  const int bs = rest / groups;  // b * s_q + s
  const int b = bs / p.s_q;
  const int s = bs - b * p.s_q;
  const int h0 = hg * kHeads;
  // this workgroup's part of the list: blocks n_begin .. n_begin + nblocks - 1
  // (none when the cache has no rows: no entry can name one)
  const int nblocks_all = p.num_rows > 0 ? (p.topk + kBlock - 1) / kBlock : 0;
  const int n_begin = split * p.blocks_per_split;
  const int nblocks = max(0, min(nblocks_all - n_begin, p.blocks_per_split));
  // entries of this part: positions 0 .. lim-1 of idx_row
  const int32_t* idx_row = p.indices + (int64_t)bs * p.topk + (int64_t)n_begin * kBlock;
  const int lim = min(p.topk - n_begin * kBlock, nblocks * kBlock);

  // ---- prologue: Q to registers --------------------------------------------------
  v4i qreg[18];  // B operand of S^T = K.Q^T: head 16w + c16, dims 32*ks + 8*G .. +7
  {
    const uint16_t* qp = p.q + ((int64_t)bs * p.h_q + h0 + wave * 16 + c16) * kDimK + 8 * G;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qreg[ks] = *reinterpret_cast<const v4i*>(qp + 32 * ks);
    // complete here: inside the loop the only loads in flight are the
    // direct-to-LDS ones, whose waits are counted exactly
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) asm volatile("" : "+v"(qreg[ks]));
  }
  if (tid == 0) {
    rescale_lds[0] = 0;
    rescale_lds[1] = 0;
    rescale_lds[2] = 0;
  }

  const uint32_t k_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)k_lds);
  const uint32_t stage_base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)stage_lds) + (uint32_t)(wave * kWaveStage);
  const uint32_t rows_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)rows_lds);
  // A token's entry is valid when it lies in this part and names a cache row.
  auto valid = [&](int pos, int r) { return pos < lim && (unsigned)r < (unsigned)p.num_rows; };
  // Row ids of block k into ring slot k % kRowRing.  Every wave loads the same
  // 32 entries (so each can wait for its own copy); positions past the part
  // read its last entry and are never used.
  auto load_rows = [&](int k, int ln) {
    const int pos = min(k * kBlock + ln, lim - 1);
    if (ln < kBlock) dma_lds4(idx_row + pos, rows_base + (uint32_t)((k % kRowRing) * kBlock * 4));
  };
  // Rows of block k into this wave's staging region (the same number of loads
  // for every block, so that waits can count them; an entry that names no row
  // loads row 0, which exists whenever there is a block).  Each wave stages and
  // dequantises its own tokens, so its region needs no barrier between uses.
  auto stage_block = [&](int k, int ln) {
    const int32_t* ring = rows_lds + (k % kRowRing) * kBlock;
    const int pp = ln & 15;
#pragma unroll
    for (int st = 0; st < kSets; ++st) {
      const int t = (wave * kSets + st) * 4 + (ln >> 4);
      const int r = ring[t];
      const uint8_t* src = p.kv + (int64_t)(valid(k * kBlock + t, r) ? r : 0) * kRowBytes;
      const uint32_t dst = stage_base + (uint32_t)(st * 3 * kRound);
      dma_lds16(src + 16 * pp, dst);
      dma_lds16(src + 256 + 16 * pp, dst + kRound);
      dma_lds16(src + kDimV + 16 * min(pp, 8), dst + 2 * kRound);
    }
  };
  // Dequantise block k from the staging region into K tile k % 3: lane (tl, p)
  // converts codes 128j + 8p .. +7 (tile j = 0..3) of its token and writes them
  // as 16 bytes of bfloat16 at 256j + 16p of the token's row, so the 16 lanes
  // of a token write 256 consecutive bytes per instruction; lanes p = 1..8
  // copy the 64 bfloat16 values.  An entry that names no row was staged from
  // row 0, which may hold anything: its K/V values are written as zeros, so
  // that its zero probability cannot meet a NaN or infinity in the products.
  auto dequant = [&](int k, int ln) {
    const uint8_t* sb = stage_lds + wave * kWaveStage;
    uint8_t* kt = k_lds + (k % kKTiles) * kKTile;
    const int32_t* ring = rows_lds + (k % kRowRing) * kBlock;
    const int tl = ln >> 4;
    const int pp = ln & 15;
#pragma unroll
    for (int st = 0; st < kSets; ++st) {
      const int t = (wave * kSets + st) * 4 + tl;
      const bool ok = valid(k * kBlock + t, ring[t]);
      const uint8_t* rb = sb + st * 3 * kRound + 256 * tl;
      uint8_t* dst = kt + krow(t) * kKStride;
      // every read first, then the conversions
      v2i codes[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        codes[j] = *reinterpret_cast<const v2i*>(rb + (j >> 1) * kRound + 128 * (j & 1) + 8 * pp);
      const v4f sc4 = *reinterpret_cast<const v4f*>(rb + 2 * kRound);
      const v4i rope = *reinterpret_cast<const v4i*>(rb + 2 * kRound + 16 * pp);
      // A power-of-two descale in [2^-100, 2^100] (the format's own: amax/448
      // rounded up to a power of two) makes code * descale exact in bfloat16,
      // and v_cvt_scalef32_pk_bf16_fp8, which applies only the scale's
      // exponent, then gives the same bits as the fp32 product rounded to
      // bfloat16, in one instruction per two values instead of four.  Other
      // descales take the fp32 product; the choice is made per wave.
      bool pow2 = true;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t su = __float_as_uint(sc4[j]);
        pow2 = pow2 && (su & 0x807fffffu) == 0 && (su >> 23) >= 27 && (su >> 23) <= 227;
      }
      const bool all_pow2 = __builtin_amdgcn_ballot_w64(!(ok && !pow2)) == ~0ull;
      // One branch around all four tiles (a branch per tile splits the
      // scheduler's regions four times).
      if (all_pow2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float scale = ok ? sc4[j] : 1.0f;
          const v2i c2 = ok ? codes[j] : v2i{0, 0};
          uint32_t w[4];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t c = (uint32_t)c2[h];
            w[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, scale, false));
            w[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, scale, true));
          }
          *reinterpret_cast<v4i*>(dst + 256 * j + 16 * pp) = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float scale = ok ? sc4[j] : 1.0f;
          const v2i c2 = ok ? codes[j] : v2i{0, 0};
          uint32_t w[4];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t c = (uint32_t)c2[h];
            const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(c, false);
            const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(c, true);
            w[2 * h] = pack_bf16(lo[0] * scale, lo[1] * scale);
            w[2 * h + 1] = pack_bf16(hi[0] * scale, hi[1] * scale);
          }
          *reinterpret_cast<v4i*>(dst + 256 * j + 16 * pp) = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
        }
      }
      if (pp >= 1 && pp <= 8)
        *reinterpret_cast<v4i*>(dst + 2 * kDimV + 16 * (pp - 1)) = ok ? rope : v4i{0, 0, 0, 0};
    }
  };

  v4f oacc[kDB][NW];  // dims kDW*w + 16*db + 4G .. +3, head 16*hb + c16
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int hb = 0; hb < NW; ++hb) oacc[db][hb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY;  // reference maximum per head (column c16 of this wave), log2 domain
  float l_run = 0.0f;       // this lane's share of the row sum, relative to the reference

  // Step n (n = 0 .. nblocks) runs, with one barrier at its end:
  //   Q.K^T of block n (K tile n % 3) beside the dequantisation of block n+1
  //   (into K tile (n+1) % 3, from this wave's staging region), then
  //   P.V of block n-1 (K tile (n-1) % 3, P buffer (n-1) & 1) beside the
  //   softmax of block n (into P buffer n & 1).
  // Loads of a wave per step: the row ids of block n+3 at the start, the rows
  // of block n+2 once its staging region has been read.  A K tile is rewritten
  // two steps after its Q.K^T and one after its P.V, a P buffer one step after
  // its P.V, so the end-of-step barrier orders every reuse.
  if (nblocks > 0) {
    load_rows(0, lane);
    load_rows(1, lane);
    load_rows(2, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    stage_block(0, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    dequant(0, lane);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the staging region has been read
    stage_block(1, lane);
  }
  lds_barrier();  // K tile 0 and the flags are ready

  // The first step has no P.V and the last no Q.K^T or softmax; the steps
  // between have both, as straight-line code that the scheduler can
  // interleave.
  auto step = [&](int n, auto qk_tag, auto pv_tag) __attribute__((always_inline)) {
    constexpr bool QK = decltype(qk_tag)::value;
    constexpr bool PV = decltype(pv_tag)::value;
    // Lane-derived offsets are recomputed every block from a lane id made
    // afresh (an opaque instruction, not a copy of `lane`), so that none of
    // them is held, in registers or spilled, across the loop.
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    load_rows(n + 3, ln);  // ring slot of block n-3, last read in step n-3
    if (tid == 0) rescale_lds[(n + 1) % 3] = 0;  // written in step n+1; last read in step n-1
    const int lG = ln >> 4;
    const int lc16 = ln & 15;

    // ---- S^T = K . Q^T for heads 16w..16w+15 ------------------------------------
    // accumulator row m of the first product is K tile row m (tokens 8(m/4) + m%4),
    // of the second row 16 + m (those + 4); lane (G, c16) then holds tokens
    // 8G .. 8G+7 of head c16 in sacc[0][0..3], sacc[1][0..3].
    v4f sacc[2] = {v4f{0.0f, 0.0f, 0.0f, 0.0f}, v4f{0.0f, 0.0f, 0.0f, 0.0f}};
    if constexpr (QK) {
      const uint8_t* kt = k_lds + (n % kKTiles) * kKTile;
      // operands read kAhead k-steps before their products
      constexpr int kAhead = 2;
      const uint8_t* a0 = kt + lc16 * kKStride + 16 * lG;
      const uint8_t* a1 = a0 + 16 * kKStride;
      v4i ka[kAhead], kb[kAhead];
#pragma unroll
      for (int i = 0; i < kAhead; ++i) {
        ka[i] = *reinterpret_cast<const v4i*>(a0 + 64 * i);
        kb[i] = *reinterpret_cast<const v4i*>(a1 + 64 * i);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);  // the first kAhead steps' reads
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        const v4i xa = ka[ks % kAhead];
        const v4i xb = kb[ks % kAhead];
        if (ks + kAhead < 18) {
          ka[ks % kAhead] = *reinterpret_cast<const v4i*>(a0 + 64 * (ks + kAhead));
          kb[ks % kAhead] = *reinterpret_cast<const v4i*>(a1 + 64 * (ks + kAhead));
        }
        sacc[0] = mfma_bf16(xa, qreg[ks], sacc[0]);
        sacc[1] = mfma_bf16(xb, qreg[ks], sacc[1]);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // the two products of step ks
        if (ks + kAhead < 18) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // reads of step ks + kAhead
      }
    }
    // ---- dequantise block n+1 ------------------------------------------------------
    // the rows of block n+1 and the row ids of n+2 (issued in the previous
    // step) are complete once only this step's row-id load is in flight
    asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    if (n + 1 < nblocks) dequant(n + 1, ln);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the staging region has been read
    stage_block(n + 2, ln);

    // ---- O^T += V^T . P^T of block n-1 for this wave's dims, all heads ---------
    if constexpr (PV) {
      const int np = n - 1;
      if (rescale_lds[np % 3]) {  // uniform; rare once the references have settled
#pragma unroll
        for (int hb = 0; hb < NW; ++hb) {
          const float al = alpha_lds[(np & 1) * kHeads + 16 * hb + lc16];
#pragma unroll
          for (int db = 0; db < kDB; ++db) oacc[db][hb] *= al;
        }
      }
      const uint8_t* kt = k_lds + (np % kKTiles) * kKTile;
      const uint8_t* pbuf = p_lds + (np & 1) * (4 * kHeads * 16);
      // transposing reads: source lane (G, j) addresses token 8G + j/4 (K tile
      // row 4G + j/4) and that token + 4 (row 16 + 4G + j/4), dims d0 + 4*(j%4);
      // result lane (G, i) then holds dim d0 + i of tokens 8G .. 8G+7
      const uint8_t* vbase = kt + (4 * lG + (lc16 >> 2)) * kKStride + 2 * (kDW * wave + 4 * (lc16 & 3));
      constexpr int kHChunk = 2;  // head blocks whose P operands are held at once
      // the wave's V operands are read once and held for every head chunk
      v4i va[kDB];
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vbase + 2 * 16 * db));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vbase + 16 * kKStride + 2 * 16 * db));
        const v2i l2 = __builtin_bit_cast(v2i, lo);
        const v2i h2 = __builtin_bit_cast(v2i, hi);
        va[db] = v4i{l2[0], l2[1], h2[0], h2[1]};
      }
#pragma unroll
      for (int h0b = 0; h0b < NW; h0b += kHChunk) {
        v4i pb[kHChunk];
#pragma unroll
        for (int j = 0; j < kHChunk; ++j)
          pb[j] = *reinterpret_cast<const v4i*>(pbuf + (lG * kHeads + 16 * (h0b + j) + lc16) * 16);
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int j = 0; j < kHChunk; ++j) oacc[db][h0b + j] = mfma_bf16(va[db], pb[j], oacc[db][h0b + j]);
      }
    }
    // ---- online softmax of block n for head c16 over tokens 8G..8G+7 -------------
    if constexpr (QK) {
      const int32_t* ring = rows_lds + (n % kRowRing) * kBlock;
      const v4i rv0 = *reinterpret_cast<const v4i*>(ring + 8 * lG);
      const v4i rv1 = *reinterpret_cast<const v4i*>(ring + 8 * lG + 4);
      const int pos0 = n * kBlock + 8 * lG;
      float x[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[r] = valid(pos0 + r, rv0[r]) ? sacc[0][r] * p.score_scale : -INFINITY;
        x[4 + r] = valid(pos0 + 4 + r, rv1[r]) ? sacc[1][r] * p.score_scale : -INFINITY;
      }
      float bmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      bmax = max_over_groups(bmax);
      // lazy reference: moved only when the block's maximum passes it by more
      // than kLazyRescale (always on the first valid block, where O is still 0)
      const bool move = bmax > m_run + kLazyRescale;
      const float m_new = move ? bmax : m_run;
      const float m_safe = m_new == -INFINITY ? 0.0f : m_new;
      const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_safe) : 1.0f;  // 0 while nothing was seen
      float e[8];
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        e[i] = __builtin_amdgcn_exp2f(x[i] - m_safe);
        sum += e[i];
      }
      const bool had = m_run != -INFINITY;
      l_run = l_run * alpha + sum;
      m_run = m_new;
      const v4i pk = v4i{(int)pack_bf16(e[0], e[1]), (int)pack_bf16(e[2], e[3]), (int)pack_bf16(e[4], e[5]),
                         (int)pack_bf16(e[6], e[7])};
      *reinterpret_cast<v4i*>(p_lds + (n & 1) * (4 * kHeads * 16) + (lG * kHeads + wave * 16 + lc16) * 16) = pk;
      if (lG == 0) alpha_lds[(n & 1) * kHeads + wave * 16 + lc16] = alpha;
      if (lG == 0 && move && had) rescale_lds[n % 3] = 1;  // accumulated O must follow the new reference
    }
    lds_barrier();  // K tile n+1, P of block n, its factors and flag are ready; tile n-1 is free
  };
  if (nblocks > 0) {
    step(0, std::true_type{}, std::false_type{});
    for (int n = 1; n < nblocks; ++n) step(n, std::true_type{}, std::true_type{});
    step(nblocks, std::false_type{}, std::true_type{});
  }

  // ---- epilogue ----------------------------------------------------------------
  const float l_tot = sum_over_groups(l_run);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load left in flight when the workgroup ends
  __syncthreads();
  if (G == 0) l_lds[wave * 16 + c16] = l_tot;
  __syncthreads();
  if (p.num_splits > 1) {
    // partial result of this part: O normalised by its own sum, and its
    // log2-sum-exp (-inf when the part selected nothing)
    const int64_t row0 = ((int64_t)split * p.B * p.s_q + bs) * p.h_q + h0;
    if (G == 0) {
      const bool empty = !(l_tot > 0.0f);
      p.lpart[row0 + wave * 16 + c16] = empty ? -INFINITY : m_run + log2f(l_tot);
    }
#pragma unroll
    for (int hb = 0; hb < NW; ++hb) {
      const float l = l_lds[16 * hb + c16];
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
      float* op = p.opart + (row0 + 16 * hb + c16) * kDimV + kDW * wave + 4 * G;
#pragma unroll
      for (int db = 0; db < kDB; ++db) *reinterpret_cast<v4f*>(op + 16 * db) = oacc[db][hb] * inv;
    }
    return;
  }
  if (p.lse != nullptr && G == 0) {
    const bool empty = !(l_tot > 0.0f);
    p.lse[((int64_t)b * p.h_q + h0 + wave * 16 + c16) * p.s_q + s] =
        empty ? kNegFltMax : (m_run + log2f(l_tot)) * kLn2;
  }
#pragma unroll
  for (int hb = 0; hb < NW; ++hb) {
    const float l = l_lds[16 * hb + c16];
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    uint16_t* op = p.out + ((int64_t)bs * p.h_q + h0 + 16 * hb + c16) * kDimV + kDW * wave + 4 * G;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      const v4f o = oacc[db][hb] * inv;
      *reinterpret_cast<v2i*>(op + 16 * db) = v2i{(int)pack_bf16(o[0], o[1]), (int)pack_bf16(o[2], o[3])};
    }
  }
}

constexpr int kMaxSplits = BSA_DECODE_MAX_SPLITS;

// Merge the parts of each (query token, head): with lse_s the parts' log2-sum-
// exp and M their maximum, O = sum_s 2^(lse_s - M) O_s / sum_s 2^(lse_s - M)
// and LSE = ln2 * (M + log2 sum_s 2^(lse_s - M)).  One workgroup of 128 threads
// per row: the weights go through LDS, then each thread sums 4 output dims
// over the parts.
__global__ void __launch_bounds__(128) bsa_fp8_decode_combine_kernel(DecodeParams p) {
  __shared__ float w_lds[kMaxSplits];
  __shared__ float max_lds[2];
  const int64_t row = blockIdx.x;  // (b * s_q + s) * h_q + h
  const int64_t rows = (int64_t)p.B * p.s_q * p.h_q;
  const int tid = threadIdx.x;
  const int S = p.num_splits;
  float mx = -INFINITY;
  for (int sp = tid; sp < S; sp += 128) {
    const float l = p.lpart[sp * rows + row];
    w_lds[sp] = l;
    mx = fmaxf(mx, l);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((tid & 63) == 0) max_lds[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(max_lds[0], max_lds[1]);
  if (mx != -INFINITY)
    for (int sp = tid; sp < S; sp += 128) w_lds[sp] = __builtin_amdgcn_exp2f(w_lds[sp] - mx);  // 0: empty part
  __syncthreads();

  const int d0 = 4 * tid;
  v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  float wsum = 0.0f;
  if (mx != -INFINITY) {
    // eight parts' loads in flight at a time: the pass is bound by reading the partials
    constexpr int kBatch = 8;
    for (int sp0 = 0; sp0 < S; sp0 += kBatch) {
      v4f o[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int sp = min(sp0 + i, S - 1);
        o[i] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p.opart + (sp * rows + row) * kDimV + d0));
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const float w = sp0 + i < S ? w_lds[sp0 + i] : 0.0f;
        wsum += w;
        acc += w * o[i];
      }
    }
  }
  const int bs = (int)(row / p.h_q);
  const int h = (int)(row - (int64_t)bs * p.h_q);
  const int b = bs / p.s_q;
  const int s = bs - b * p.s_q;
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  const v4f o = acc * inv;
  *reinterpret_cast<v2i*>(p.out + row * kDimV + d0) = v2i{(int)pack_bf16(o[0], o[1]), (int)pack_bf16(o[2], o[3])};
  if (p.lse != nullptr && tid == 0)
    p.lse[((int64_t)b * p.h_q + h) * p.s_q + s] = wsum > 0.0f ? (mx + log2f(wsum)) * kLn2 : kNegFltMax;
}


int64_t partial_rows(const bsa_fp8_decode_dims& d) { return (int64_t)d.batch * d.s_q * d.num_heads_q; }

// Static checks shared by the split-list entry points; sets *grid (decode
// workgroups) and returns BSA_OK, or the first error found.
int validate(const void* q, const void* kv_cache, const int32_t* indices, const bsa_fp8_decode_dims* dims,
             int num_splits, const void* out, int64_t* grid) {
  if (dims == nullptr) return BSA_ERR_NULL_POINTER;
  const bsa_fp8_decode_dims d = *dims;
  if (d.batch < 0 || d.s_q < 0 || d.num_heads_q <= 0 || d.topk <= 0 || d.num_pages < 0) return BSA_ERR_SIZE;
  if (d.num_heads_q % 64 != 0) return BSA_ERR_GQA;
  if (num_splits < 1 || num_splits > kMaxSplits) return BSA_ERR_SIZE;
  const int nblocks_all = (d.topk + kBlock - 1) / kBlock;
  const int bps = (nblocks_all + num_splits - 1) / num_splits;
  if ((int64_t)bps * kBlock > kMaxTopk) return BSA_ERR_TOO_LARGE;  // a part longer than the interface allows
  if (d.page_size <= 0) return BSA_ERR_PAGE_SIZE;
  if (!bsa::finite_float(d.softmax_scale)) return BSA_ERR_SOFTMAX_SCALE;
  const int nw = d.num_heads_q % 128 == 0 ? 8 : 4;  // 16 heads per wave
  const int64_t g = (int64_t)d.batch * d.s_q * (d.num_heads_q / (16 * nw)) * num_splits;
  if (g > 0x7fffffffLL) return BSA_ERR_TOO_LARGE;
  if ((int64_t)d.num_pages * d.page_size > 0x7fffffffLL) return BSA_ERR_TOO_LARGE;  // 32-bit row ids
  if (num_splits > 1 && partial_rows(d) > 0x7fffffffLL) return BSA_ERR_TOO_LARGE;
  *grid = g;
  if (g == 0) return BSA_OK;
  if (q == nullptr || kv_cache == nullptr || indices == nullptr || out == nullptr) return BSA_ERR_NULL_POINTER;
  return BSA_OK;
}

// Enqueue the decode (and, for several parts, the merge) with `ws` holding
// the partial results.
int launch(const void* q, const void* kv_cache, const int32_t* indices, const bsa_fp8_decode_dims& d,
           int num_splits, float* ws, void* out, float* lse, void* stream, int64_t grid) {
  const int nblocks_all = (d.topk + kBlock - 1) / kBlock;
  const int bps = (nblocks_all + num_splits - 1) / num_splits;
  const int nw = d.num_heads_q % 128 == 0 ? 8 : 4;
  DecodeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.kv = static_cast<const uint8_t*>(kv_cache);
  p.indices = indices;
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.B = d.batch;
  p.s_q = d.s_q;
  p.h_q = d.num_heads_q;
  p.topk = d.topk;
  p.num_rows = d.num_pages * d.page_size;
  p.score_scale = d.softmax_scale * kLog2e;
  p.num_splits = num_splits;
  p.blocks_per_split = bps;
  p.opart = ws;
  p.lpart = num_splits > 1 ? p.opart + (int64_t)num_splits * partial_rows(d) * kDimV : nullptr;
  if (nw == 8)
    hipLaunchKernelGGL(bsa_fp8_decode_kernel<8>, dim3((unsigned)grid), dim3(512), 0,
                       static_cast<hipStream_t>(stream), p);
  else
    hipLaunchKernelGGL(bsa_fp8_decode_kernel<4>, dim3((unsigned)grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), p);
  if (num_splits > 1)
    hipLaunchKernelGGL(bsa_fp8_decode_combine_kernel, dim3((unsigned)partial_rows(d)), dim3(128), 0,
                       static_cast<hipStream_t>(stream), p);
  if (hipGetLastError() != hipSuccess) return BSA_ERR_LAUNCH;
  return BSA_OK;
}

// Partial results of bsa_fp8_sparse_decode_noalloc: a file-scope device array,
// one copy per GPU for the life of the process.  Host code never passes its
// name to a kernel (on the host the name is only a stand-in); it uses the
// device address that hipGetSymbolAddress returns for the current device,
// looked up once per device on the first call there.
constexpr uint64_t kScratchBytes = BSA_DECODE_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(float** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BSA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || a == nullptr) return BSA_ERR_LAUNCH;
    g_scratch_ptr[dev] = static_cast<float*>(a);
  }
  *ptr = g_scratch_ptr[dev];
  return BSA_OK;
}

// Part count for the no-allocation entry point: the library's choice, lowered
// until the partial results fit the scratch (never below the parts a list
// needs; validation then reports what does not fit).
int noalloc_splits(const bsa_fp8_decode_dims& d) {
  int n = bsa_fp8_sparse_decode_num_splits(&d);
  const uint64_t per_part = (uint64_t)partial_rows(d) * (kDimV + 1) * 4;
  const int nblocks = (d.topk + kBlock - 1) / kBlock;
  const int need = (nblocks * kBlock + kMaxTopk - 1) / kMaxTopk;  // parts whose lists fit
  while (n > 1 && n > need && (uint64_t)n * per_part > kScratchBytes) --n;
  return n;
}

}  // namespace

extern "C" {

int bsa_fp8_sparse_decode_num_splits(const bsa_fp8_decode_dims* dims) {
  if (dims == nullptr || dims->num_heads_q <= 0 || dims->num_heads_q % 64 != 0 || dims->topk <= 0) return 1;
  const int nw = dims->num_heads_q % 128 == 0 ? 8 : 4;
  const int64_t base = (int64_t)dims->batch * dims->s_q * (dims->num_heads_q / (16 * nw));
  const int nblocks = (dims->topk + kBlock - 1) / kBlock;
  // at least enough parts for the row list of each to fit; then enough
  // workgroups to occupy every CU, with at least 2 blocks per part (a sweep
  // over batch sizes 1..64 at top-k 2048 put the best count within 4% of this)
  const int need = (nblocks * kBlock + kMaxTopk - 1) / kMaxTopk;
  int64_t want = base > 0 ? (256 + base - 1) / base : 1;
  want = want < (nblocks + 1) / 2 ? want : (nblocks + 1) / 2;
  int64_t sp = want > need ? want : need;
  if (sp < 1) sp = 1;
  if (sp > kMaxSplits) sp = kMaxSplits;
  return (int)sp;
}

long long bsa_fp8_sparse_decode_workspace_bytes(const bsa_fp8_decode_dims* dims, int num_splits) {
  if (dims == nullptr || num_splits < 1 || num_splits > kMaxSplits || dims->batch < 0 || dims->s_q < 0 ||
      dims->num_heads_q <= 0)
    return -1;
  if (num_splits == 1) return 0;
  return (long long)num_splits * partial_rows(*dims) * (kDimV + 1) * 4;
}


int bsa_fp8_sparse_decode_ex(const void* q, const void* kv_cache, const int32_t* indices,
                             const bsa_fp8_decode_dims* dims, int num_splits, void* workspace, void* out,
                             float* lse, void* stream) {
  int64_t grid = 0;
  const int st = validate(q, kv_cache, indices, dims, num_splits, out, &grid);
  if (st != BSA_OK || grid == 0) return st;
  if (num_splits > 1 && workspace == nullptr) return BSA_ERR_NULL_POINTER;
  if (num_splits > 1 && reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return BSA_ERR_SIZE;
  return launch(q, kv_cache, indices, *dims, num_splits, static_cast<float*>(workspace), out, lse, stream, grid);
}

int bsa_fp8_sparse_decode_noalloc(const void* q, const void* kv_cache, const int32_t* indices,
                                  const bsa_fp8_decode_dims* dims, int num_splits, void* out, float* lse,
                                  void* stream) {
  if (dims == nullptr) return BSA_ERR_NULL_POINTER;
  if (num_splits == 0) num_splits = noalloc_splits(*dims);
  int64_t grid = 0;
  const int st = validate(q, kv_cache, indices, dims, num_splits, out, &grid);
  if (st != BSA_OK) return st;
  if (num_splits > 1 && (uint64_t)num_splits * partial_rows(*dims) * (kDimV + 1) * 4 > (uint64_t)kScratchBytes)
    return BSA_ERR_SCRATCH;
  if (grid == 0) return BSA_OK;
  float* ws = nullptr;
  if (num_splits > 1) {
    const int sst = scratch_address(&ws);
    if (sst != BSA_OK) return sst;
  }
  return launch(q, kv_cache, indices, *dims, num_splits, ws, out, lse, stream, grid);
}

int bsa_fp8_sparse_decode(const void* q, const void* kv_cache, const int32_t* indices,
                          const bsa_fp8_decode_dims* dims, void* out, float* lse, void* stream) {
  return bsa_fp8_sparse_decode_ex(q, kv_cache, indices, dims, 1, nullptr, out, lse, stream);
}

}  // extern "C"
