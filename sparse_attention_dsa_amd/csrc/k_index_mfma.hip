// Indexer score on the matrix cores, 64 heads x 128 dims, bf16 queries, bf16 or fp8 keys:
//   s[t][j] = sum_h w[t][h] * relu(q[t][h] . k_j),  j = 0 .. position(t)
// (DSA resource page: module description, index_topk.)
//
// One workgroup (4 waves) scores KPB consecutive keys of one row (two min / max blocks). Per 16-key tile a wave runs
// 16 v_mfma_f32_16x16x32_bf16: heads are M (4 tiles of 16), keys are N, dims are K (4 steps of
// 32). The row's queries stay in VGPRs as the A operand for the whole block. Keys stream from
// HBM into a ring of tiles in LDS that each wave owns, with global_load_lds: every instruction
// moves 1 KB of whole key rows (the access pattern HBM serves fastest), and the 16-byte pieces of
// a key's row are XOR-swizzled by the key so that the B-operand reads are free of bank
// conflicts. Lane l takes key l%16 and the pieces l/16, l/16 + 4, ... of its row (fp8 codes
// become bf16 exactly in registers); the A operand takes the query's dims in the same order, so
// the contraction is unchanged. The epilogue (relu, head
// weight, sum over heads) runs on the accumulators: each lane sums its 16 heads, two lane swaps
// (v_permlane16_swap / v_permlane32_swap) finish the 64. An fp8 key is e4m3(code) * scale; the
// scale is >= 0 and multiplies the finished sum (relu(c*x) = c*relu(x) for c >= 0).
// Each block also writes the min and max order key of its scores for the top-k select and, on
// request, the best order key of every 32-key group (block-sparse selection).
#include "dsa_internal.hpp"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int H = 64, D = 128;
constexpr int kQPitch = D + 8;                     // bf16 elements per q row in LDS (padded)
#ifndef DSA_INDEX_WAVES
#define DSA_INDEX_WAVES 4            // waves per workgroup
#endif
constexpr int kWaves = DSA_INDEX_WAVES;
// Keys per workgroup: two of the select's min / max blocks (fewer, longer workgroups measured
// faster at 128K contexts; the per-workgroup set-up is then paid half as often).
constexpr int kHalves = 2;
constexpr int KPB = kHalves * kScoreBlock;

template <int KFMT>
struct Raw {
  // bf16: 64 bytes of one key (4 x 16 B); fp8: 32 bytes (2 x 16 B) and the key's scale
  u32x4 v[KFMT == DSA_FMT_BF16 ? 4 : 2];
  float scale;
};

#ifndef DSA_INDEX_DEPTH_FP8
#define DSA_INDEX_DEPTH_FP8 8        // key tiles in flight per wave
#endif
#ifndef DSA_INDEX_DEPTH_BF16
#define DSA_INDEX_DEPTH_BF16 4
#endif

// A 16-key tile in a wave's LDS ring: the keys' rows (16 B pieces swizzled), then for fp8 the
// keys' scales. Each code DMA moves 1 KB: kKeysPerOp whole rows.
template <int KFMT> struct Tile;
template <> struct Tile<DSA_FMT_BF16> {
  static constexpr int kRow = 2 * D, kPieces = 16, kCodeOps = 4, kScaleBytes = 0;
  static constexpr int kDepth = DSA_INDEX_DEPTH_BF16;
  // pieces p of key k sit at p ^ k: the 16 keys of one B read (same p) hit distinct bank groups
  static __device__ __forceinline__ int swz(int k) { return k & 15; }
};
template <> struct Tile<DSA_FMT_FP8> {
  static constexpr int kRow = D, kCodeOps = 2, kScaleBytes = 64;
  [[maybe_unused]] static constexpr int kPieces = 8;   // read only by the fp8 LDS-ring variant
  static constexpr int kDepth = DSA_INDEX_DEPTH_FP8;
  // two keys share a 256-byte bank row (one per half); pieces p of key k sit at p ^ (k/2)
  static __device__ __forceinline__ int swz(int k) { return (k >> 1) & 7; }
};

__device__ __forceinline__ void dma16(const void* src, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}
// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding), then a compiler
// barrier so that no LDS read of the awaited tile is hoisted above the wait
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}
// wait_vmcnt for a count known once the caller's loop is unrolled (the switch folds away)
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define DSA_W(N) case N: wait_vmcnt<N>(); break;
    DSA_W(0) DSA_W(1) DSA_W(2) DSA_W(3) DSA_W(4) DSA_W(5) DSA_W(6) DSA_W(7) DSA_W(8) DSA_W(9)
    DSA_W(10) DSA_W(11) DSA_W(12) DSA_W(13) DSA_W(14) DSA_W(15) DSA_W(16) DSA_W(17) DSA_W(18)
    DSA_W(19) DSA_W(20) DSA_W(21) DSA_W(22) DSA_W(23) DSA_W(24) DSA_W(25) DSA_W(26) DSA_W(27)
    DSA_W(28) DSA_W(29) DSA_W(30) DSA_W(31)
#undef DSA_W
    default: wait_vmcnt<0>(); break;
  }
}
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}
__device__ __forceinline__ u32x4 lds_b128(uint32_t at) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(uintptr_t(at));
}
__device__ __forceinline__ float lds_f32(uint32_t at) {
  return *reinterpret_cast<const __attribute__((address_space(3))) float*>(uintptr_t(at));
}

// max(x, 0) as one integer max on the bit pattern: positive floats are positive integers, and
// negative floats (-0 included) are negative integers and become +0.
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// B fragment for k-step ks of the lane's key: bf16 dims 32*ks + 8*grp .. +8; fp8 dims
// 64*(ks/2) + 16*grp + 8*(ks%2) .. +8 (the A operand takes the query's dims in the same order).
template <int KFMT>
__device__ __forceinline__ bf16x8 b_frag(const Raw<KFMT>& r, int ks) {
  if constexpr (KFMT == DSA_FMT_BF16) {
    return __builtin_bit_cast(bf16x8, r.v[ks]);
  } else {
    const uint32_t lo = r.v[ks >> 1][(ks & 1) * 2], hi = r.v[ks >> 1][(ks & 1) * 2 + 1];
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    const bf16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    const bf16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

#ifndef DSA_INDEX_WAVES_PER_SIMD
#define DSA_INDEX_WAVES_PER_SIMD 2   // register budget: 512 / this VGPRs per lane
#endif

#ifndef DSA_INDEX_DMA_FP8
#define DSA_INDEX_DMA_FP8 0          // fp8 keys through the LDS ring (0: straight into registers)
#endif
#ifndef DSA_INDEX_DMA_BF16
#define DSA_INDEX_DMA_BF16 1
#endif
#ifndef DSA_INDEX_VDEPTH
#define DSA_INDEX_VDEPTH 8           // tiles in flight per wave when keys go straight to registers
#endif

// Loads one tile's share for this lane straight into registers: key j (request-local), the
// 16-byte pieces grp, grp + 4, ... of the key's row (64 contiguous bytes of every key per load).
template <int KFMT, bool OFF32>
__device__ __forceinline__ void load_tile(Raw<KFMT>& r, const uint8_t* pool,
                                          const uint32_t* __restrict__ base_lds, int first_list,
                                          int page_start, int log2_ps, int ps_mask, int64_t page_bytes,
                                          int j, int lane_grp) {
  const int slot = page_start + j;
  const uint32_t b = base_lds[(slot >> log2_ps) - first_list];
  const uint32_t off = uint32_t(slot & ps_mask);
  constexpr uint32_t kRow = Tile<KFMT>::kRow;
  const uint32_t in_page = off * kRow + uint32_t(lane_grp) * 16u;
  const uint32_t scale_at = (uint32_t(ps_mask) + 1) * D + off * 4;
  const u32x4* src;
  const float* sc;
  if constexpr (OFF32) {
    src = reinterpret_cast<const u32x4*>(pool + (b + in_page));
    sc = reinterpret_cast<const float*>(pool + (b + scale_at));
  } else {
    const uint8_t* pg = pool + int64_t(b) * page_bytes;
    src = reinterpret_cast<const u32x4*>(pg + in_page);
    sc = reinterpret_cast<const float*>(pg + scale_at);
  }
  if constexpr (KFMT == DSA_FMT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[i] = __builtin_nontemporal_load(src + 4 * i);
    r.scale = 1.0f;
  } else {
    r.v[0] = __builtin_nontemporal_load(src);
    r.v[1] = __builtin_nontemporal_load(src + 4);
    r.scale = *sc;
  }
}

// fp8 keys as whole rows: the two load instructions of a 16-key tile read 1 KB each, keys 0-7
// and keys 8-15 of the tile (8 whole 128-byte rows), which the memory system serves faster than
// the 64-byte halves of 16 rows. Lane l (key c = l % 16, B-operand pieces g = l / 16 and g + 4)
// loads, in instruction 0, piece g of key c when c < 8 and else piece g + 4 of key c - 8; in
// instruction 1, piece g + 4 of key c + 8 when c < 8 and else piece g of key c. fp8_rows_fix
// then hands every piece loaded for the partner lane l ^ 8 over (a DPP rotate by 8 inside each
// row of 16 lanes), so that r.v = {piece g, piece g + 4} of key c. k0 and k1 are the keys of the
// two instructions and p0, p1 their pieces (request-local keys, clamped into the row); the scale
// is key c's.
template <bool OFF32>
__device__ __forceinline__ void load_rows_fp8(Raw<DSA_FMT_FP8>& r, const uint8_t* pool,
                                              const uint32_t* __restrict__ base_lds, int first_list,
                                              int page_start, int log2_ps, int ps_mask, int64_t page_bytes,
                                              int k0, int k1, uint32_t p0, uint32_t p1, bool low_half) {
  const int s0 = page_start + k0, s1 = page_start + k1;
  const uint32_t b0 = base_lds[(s0 >> log2_ps) - first_list];
  const uint32_t b1 = base_lds[(s1 >> log2_ps) - first_list];
  const uint32_t o0 = uint32_t(s0 & ps_mask), o1 = uint32_t(s1 & ps_mask);
  const uint32_t bs = low_half ? b0 : b1, os = low_half ? o0 : o1;
  const uint32_t in0 = o0 * uint32_t(D) + p0 * 16u, in1 = o1 * uint32_t(D) + p1 * 16u;
  const uint32_t scale_at = (uint32_t(ps_mask) + 1) * D + os * 4;
  const uint8_t *src0, *src1, *sc;
  if constexpr (OFF32) {
    src0 = pool + (b0 + in0);
    src1 = pool + (b1 + in1);
    sc = pool + (bs + scale_at);
  } else {
    src0 = pool + int64_t(b0) * page_bytes + in0;
    src1 = pool + int64_t(b1) * page_bytes + in1;
    sc = pool + int64_t(bs) * page_bytes + scale_at;
  }
  r.v[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src0));
  r.v[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src1));
  r.scale = *reinterpret_cast<const float*>(sc);
}

// The tile as load_rows_fp8 left it -> the B-operand layout (pieces g and g + 4 of key l % 16)
__device__ __forceinline__ Raw<DSA_FMT_FP8> fp8_rows_fix(const Raw<DSA_FMT_FP8>& r, bool low_half) {
  Raw<DSA_FMT_FP8> o;
  o.scale = r.scale;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    o.v[0][c] = low_half ? r.v[0][c] : r.v[1][c];
    const uint32_t give = low_half ? r.v[1][c] : r.v[0][c];
    // row_ror:8: lane i of each 16-lane row takes lane (i + 8) mod 16
    o.v[1][c] = uint32_t(__builtin_amdgcn_mov_dpp(int(give), 0x128, 0xF, 0xF, false));
  }
  return o;
}

// MODE kRuns: also write the best order key of every 32-key group to run_max (block-sparse
// selection). MODE kHist: also write the block's fixed-bin histogram (ScoreHist) for the fused
// select. Separate instantiations, so that the plain kernel's code is untouched.
constexpr int kPlain = 0, kRuns = 1, kHist = 2;
static_assert(ScoreHist::kBlock == kHalves * kScoreBlock, "a histogram block is a score workgroup");

template <int KFMT, bool OFF32, int MODE>
__global__ void __launch_bounds__(kWaves * 64, DSA_INDEX_WAVES_PER_SIMD)
index_scores_mfma(DevPlan p, RowMap map, const uint16_t* __restrict__ q, const float* __restrict__ w,
                  const uint8_t* pool, float* __restrict__ scores, int64_t ld,
                  int64_t page_bytes, int log2_ps, uint32_t* __restrict__ blk_minmax, int nb_max,
                  int fill_masked, uint32_t* __restrict__ run_max, int64_t rm_ld, ScoreHist hist) {
  constexpr bool RUNS = MODE == kRuns;
  using TL = Tile<KFMT>;
  constexpr bool FP8 = KFMT == DSA_FMT_FP8;
  constexpr bool DMA = FP8 ? DSA_INDEX_DMA_FP8 : DSA_INDEX_DMA_BF16;
  constexpr int kDepth = DMA ? TL::kDepth : DSA_INDEX_VDEPTH;
  constexpr int kTileBytes = 16 * TL::kRow + TL::kScaleBytes;
  constexpr int kOps = TL::kCodeOps + (FP8 ? 1 : 0);       // vector-memory ops per DMA tile
  static_assert(kDepth % 4 == 0, "whole runs per ring pass");
  // the waves' LDS rings (DMA); the row's queries are staged here first. Per page of the block,
  // its pool byte offset (OFF32) or id.
  constexpr int kQBytes = H * kQPitch * 2;
  constexpr int kRingBytes = DMA ? kWaves * kDepth * kTileBytes : 0;
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRingBytes > kQBytes ? kRingBytes : kQBytes];
  __shared__ uint32_t red[2 * kHalves * kWaves];
  __shared__ uint32_t s_wsum[kWaves], s_c;
  // sized at launch: KPB / page_size + 2 page entries (rounded up to 16 bytes); kHist then keeps
  // the block's KPB scores here for the epilogue instead of writing them to HBM
  extern __shared__ uint32_t pages_lds[];
  float* s_sc = reinterpret_cast<float*>(pages_lds + ((KPB >> log2_ps) + 2 + 3) / 4 * 4);
  uint16_t* q_lds = reinterpret_cast<uint16_t*>(ring);

  // step row of this launch index: ranges of consecutive rows, a handful at most
  const int li = blockIdx.y;
  int mr = 0;
  while (mr + 1 < map.n && map.first[mr + 1] <= li) ++mr;
  const int t = map.start[mr] + (li - map.first[mr]);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4, col = lane & 15;

  // the row's span heads the chain (span -> page ids -> keys) and goes first; then the head weights
  // of the accumulator rows this lane holds (head 16*mt + 4*grp + v), whose latency overlaps the
  // lookups below (the span lookup waits for the span's load only)
  const dsa_span span0 = dsa::span_chunk(p.spans, p.n_spans, 0);
  asm volatile("" ::: "memory");
  float wr[16];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) wr[mt * 4 + v] = w[int64_t(t) * H + 16 * mt + 4 * grp + v];

  dsa_span sp;
  dsa::row_span_from(span0, p.spans, p.n_spans, t, &sp);
  const int pos = sp.ctx_start + (t - sp.q_start);
  const int n = pos + 1;
  const int kb = blockIdx.x * KPB;
  float* out = scores + int64_t(t) * ld;

  if (kb >= n) {
    if (fill_masked)
      for (int j = kb + threadIdx.x; j < ld && j < kb + KPB; j += kWaves * 64) out[j] = -__builtin_inff();
    return;
  }
  const int ps_mask = (1 << log2_ps) - 1;
  const int kend = min(n, kb + KPB);
  const int first_list = (sp.page_start + kb) >> log2_ps;
  const int last_list = (sp.page_start + kend - 1) >> log2_ps;

  // Stage this block's page ids and the row's queries (whole 16-byte pieces, coalesced) in LDS.
  // The page ids are requested first: the keys wait for them, while the queries are needed only
  // when the first tile is in.
  for (int i = threadIdx.x; i <= last_list - first_list; i += kWaves * 64) {
    int pg = p.page_table[dsa::page_entry(sp, first_list + i)];
    pg = pg < 0 ? 0 : (pg >= p.pool_pages ? p.pool_pages - 1 : pg);
    pages_lds[i] = OFF32 ? uint32_t(int64_t(pg) * page_bytes) : uint32_t(pg);
  }
  constexpr int kQPieces = H * D / 8 / (kWaves * 64);     // 16-byte query pieces per thread
  u32x4 qv[kQPieces];
  {
    const u32x4* qs = reinterpret_cast<const u32x4*>(q + int64_t(t) * H * D);
#pragma unroll
    for (int i = 0; i < kQPieces; ++i) qv[i] = qs[threadIdx.x + kWaves * 64 * i];
  }
  auto store_q = [&]() {
#pragma unroll
    for (int i = 0; i < kQPieces; ++i) {
      const int e = threadIdx.x + kWaves * 64 * i, h = e / (D / 8), c = e % (D / 8);
      *reinterpret_cast<u32x4*>(q_lds + h * kQPitch + c * 8) = qv[i];
    }
  };
  bf16x8 a[4][4];
  // A operand: head 16*mt + col, the same 8 dims as the B fragment of k-step ks
  auto read_a = [&]() {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int d0 = FP8 ? 64 * (ks >> 1) + 16 * grp + 8 * (ks & 1) : 32 * ks + 8 * grp;
        a[mt][ks] = *reinterpret_cast<const bf16x8*>(q_lds + (16 * mt + col) * kQPitch + d0);
      }
  };
  if constexpr (DMA) {
    // the ring holds the staged queries first: it starts once every wave has read them
    store_q();
    __syncthreads();
    read_a();
    // Pin the operands here so that their loads are complete before the ring starts: from now on
    // the vector-memory counter holds only this wave's DMAs and score stores, which the waits
    // count. Every wave's A operands are then read, so the ring may overwrite the queries.
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(wr[i]));
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) asm volatile("" : "+v"(a[mt][ks]));
    wait_vmcnt<0>();
    __syncthreads();
  } else {
    __syncthreads();                        // page ids staged
  }

  // score range of each half of the block
  float fmin0 = __builtin_inff(), fmax0 = -__builtin_inff();
  float fmin1 = __builtin_inff(), fmax1 = -__builtin_inff();
  // A wave works through 64-key runs of the block, run q*kWaves + wave for q = 0, 1, ...: tile
  // it of the wave is tile it%4 of its run it/4.
  auto run_of = [&](int it) { return (it >> 2) * kWaves + wave; };
  auto tile_key = [&](int it) { return kb + 64 * run_of(it) + 16 * (it & 3) + col; };

  // Q.K^T of one tile: 16 MFMAs into four accumulators (heads 16*mt + 4*grp + v, key col)
  auto mma = [&](const Raw<KFMT>& r, f32x4* acc) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 b = b_frag<KFMT>(r, ks);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt][ks], b, acc[mt], 0, 0, 0);
    }
  };
  // relu and head weights of the lane's 16 heads of one tile (two fma chains), times the key's
  // scale
  auto tile_sum = [&](const f32x4* acc, float scale) {
    float c0 = wr[0] * relu_bits(acc[0][0]);
    float c1 = wr[8] * relu_bits(acc[2][0]);
#pragma unroll
    for (int e = 1; e < 8; ++e) {
      c0 = fmaf(wr[e], relu_bits(acc[e >> 2][e & 3]), c0);
      c1 = fmaf(wr[8 + e], relu_bits(acc[2 + (e >> 2)][e & 3]), c1);
    }
    return (c0 + c1) * scale;
  };
  // The four tiles of a run: lane l holds one quarter of the heads (accumulator row l/16) of key
  // 16*tt + l%16 for each tile tt. v_permlane32_swap puts tiles 0 and 2 (1 and 3) side by side
  // with the row pairs (0,2) and (1,3) added, v_permlane16_swap adds rows 0+1 and 2+3 and
  // interleaves the tiles back into key order: lane l ends with the whole score of run key l,
  // stored with one instruction. A key past the row (loaded as key kend - 1) repeats that key's
  // score, the same bits, at the same place.
  auto finish_run = [&](const float* part, int it0) {
    const auto p02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
    const auto p13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
    const float x = __uint_as_float(p02[0]) + __uint_as_float(p02[1]);
    const float y = __uint_as_float(p13[0]) + __uint_as_float(p13[1]);
    const auto pxy = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    const float val = __uint_as_float(pxy[0]) + __uint_as_float(pxy[1]);
    const int j = min(kb + 64 * run_of(it0) + lane, kend - 1);
    out[j] = val;
    if constexpr (MODE == kHist) s_sc[j - kb] = val;
    if constexpr (RUNS) {
      // the best order key of each 32-key group of the run (keys past the row repeat the row's
      // last score, so they change no group's maximum), for block selection at that granularity
      const uint32_t k = dsa::group_max_last<32>(dsa::order_key(val));
      const int g0 = kb + 64 * run_of(it0) + (lane & 32);
      if ((lane & 31) == 31 && g0 < kend) run_max[int64_t(t) * rm_ld + (g0 >> 5)] = k;
    }
    if (64 * run_of(it0) < kScoreBlock) {
      fmin0 = fminf(fmin0, val);
      fmax0 = fmaxf(fmax0, val);
    } else {
      fmin1 = fminf(fmin1, val);
      fmax1 = fmaxf(fmax1, val);
    }
  };

  // runs of this wave that hold at least one key of the row; a ring of kDepth tiles in flight
  const int n_runs = min(KPB / 64, (kend - kb + 63) / 64);
  const int n_it = 4 * ((n_runs - wave + kWaves - 1) / kWaves);

  if constexpr (DMA) {
    // DMA of tile it into ring slot d: key k of the tile is loaded by the lanes of op
    // k / (keys per op); cell s of an op holds piece (s % P) ^ swz(k) of key k (P pieces a key).
    // Keys past the row load key kend - 1. Addresses first, then the DMAs, so that the page-id
    // reads overlap.
    const uint32_t ring_w = lds_u32(ring) + uint32_t(wave * kDepth * kTileBytes);
    auto src_of = [&](int j, uint32_t in_row) -> const uint8_t* {
      const int slot = sp.page_start + j;
      const uint32_t b = pages_lds[(slot >> log2_ps) - first_list];
      const uint32_t off = uint32_t(slot & ps_mask);
      if constexpr (OFF32) return pool + (b + off * uint32_t(TL::kRow) + in_row);
      else return pool + int64_t(b) * page_bytes + off * uint32_t(TL::kRow) + in_row;
    };
    auto issue = [&](int it, int d) {
      const int key0 = kb + 64 * run_of(it) + 16 * (it & 3);
      const uint8_t* src[kOps];
#pragma unroll
      for (int i = 0; i < TL::kCodeOps; ++i) {
        const int s = 64 * i + lane;
        const int k = s / TL::kPieces;
        const int pc = (s % TL::kPieces) ^ TL::swz(k);
        src[i] = src_of(min(key0 + k, kend - 1), uint32_t(16 * pc));
      }
      if constexpr (FP8) {
        // the page's scales follow its codes, 4 bytes a key: from the row start, the rest of the
        // page's codes and then this key's place among the scales
        const int j = min(key0 + (lane & 15), kend - 1);
        const uint32_t off = uint32_t((sp.page_start + j) & ps_mask);
        src[TL::kCodeOps] = src_of(j, (uint32_t(ps_mask) + 1 - off) * uint32_t(D) + off * 4u);
      }
      const uint32_t dst = ring_w + uint32_t(d * kTileBytes);
#pragma unroll
      for (int i = 0; i < TL::kCodeOps; ++i) dma16(src[i], dst + uint32_t(1024 * i));
      if constexpr (FP8) {
        if (lane < 16) dma4(src[TL::kCodeOps], dst + uint32_t(16 * TL::kRow));
      }
    };
    // B fragments and scale of key col of the tile in slot d: pieces grp + 4i of its row
    auto read_tile = [&](Raw<KFMT>& r, int d) {
      const uint32_t row = ring_w + uint32_t(d * kTileBytes + col * TL::kRow);
#pragma unroll
      for (int i = 0; i < TL::kPieces / 4; ++i)
        r.v[i] = lds_b128(row + uint32_t(16 * ((grp + 4 * i) ^ TL::swz(col))));
      if constexpr (FP8) r.scale = lds_f32(ring_w + uint32_t(d * kTileBytes + 16 * TL::kRow + 4 * col));
      else r.scale = 1.0f;
    };
    // DMAs are unconditional (a tile past the row reloads the row's last key), so every wait
    // counts a fixed sequence: kOps DMAs per tile and kSt = 1 score store per run of 4 tiles
    // (kRuns stores more, which only makes its waits longer). Tile it + d (slot d) is in once at
    // most the ops issued after its DMAs are outstanding: the DMAs of the next kDepth - 1 tiles and
    // the stores between. In the first pass those stores are kSt per run of tiles 0 .. d - 1;
    // afterwards the window of kDepth - 1 tiles holds kSt per run, one run fewer when it ends just
    // before a run's last tile.
    constexpr int kSt = 1;
#pragma unroll
    for (int d = 0; d < kDepth; ++d) issue(d, d);
    for (int it = 0; it < n_it; it += kDepth) {
      float part[4];
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        constexpr int kWin = kOps * (kDepth - 1);
        static_assert(kWin + kDepth / 4 < 32, "wait counts in range");
        if (it == 0) wait_vm(kWin + kSt * (d / 4));
        else wait_vm((d & 3) == 3 ? kWin + kSt * (kDepth / 4 - 1) : kWin + kSt * (kDepth / 4));
        Raw<KFMT> r;
        read_tile(r, d);
        f32x4 acc[4];
        mma(r, acc);
        part[d & 3] = tile_sum(acc, r.scale);
        if ((d & 3) == 3) finish_run(part, it + d - 3);
        issue(it + d + kDepth, d);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_vmcnt<0>();   // the ring's last DMAs land before the workgroup's LDS is released
  } else {
    // keys straight into a ring of registers; the compiler counts these loads itself
    const bool low_half = (lane & 8) == 0;
    const uint32_t p0 = uint32_t(grp) + (low_half ? 0u : 4u), p1 = uint32_t(grp) + (low_half ? 4u : 0u);
    auto load = [&](Raw<KFMT>& r, int it) {
      const int j = min(tile_key(it), kend - 1);   // keys past the row load a valid key
      if constexpr (FP8) {
        const int tb = tile_key(it) - col;          // the tile's first key (a multiple of 16 from kb)
        const int k0 = min(tb + (col & 7), kend - 1), k1 = min(tb + (col | 8), kend - 1);
        load_rows_fp8<OFF32>(r, pool, pages_lds, first_list, sp.page_start, log2_ps, ps_mask, page_bytes, k0, k1, p0, p1, low_half);
      } else {
        load_tile<KFMT, OFF32>(r, pool, pages_lds, first_list, sp.page_start, log2_ps, ps_mask, page_bytes, j, grp);
      }
    };
    Raw<KFMT> vring[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) load(vring[d], d);
    // the queries go to LDS while the first tiles are in flight (the barriers keep the tile loads
    // ahead of the query stores, which wait for the query loads; the pool is not marked
    // __restrict__ so that the compiler keeps its loads on this side of them)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    store_q();
    __syncthreads();
    read_a();
    for (int it = 0; it < n_it; it += kDepth) {
      float part[4];
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        f32x4 acc[4];
        if constexpr (FP8) {
          const Raw<KFMT> rf = fp8_rows_fix(vring[d], low_half);
          mma(rf, acc);
          part[d & 3] = tile_sum(acc, rf.scale);
        } else {
          mma(vring[d], acc);
          part[d & 3] = tile_sum(acc, vring[d].scale);
        }
        if ((d & 3) == 3) finish_run(part, it + d - 3);
        load(vring[d], it + d + kDepth);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (fill_masked)
    for (int j = kend + threadIdx.x; j < kb + KPB && j < ld; j += kWaves * 64) out[j] = -__builtin_inff();

  // min / max order key of each half (a wave with no key in it keeps the empty range); a half
  // that starts past the row has no entry (the select reads none there)
#pragma unroll
  for (int hf = 0; hf < kHalves; ++hf) {
    const float fmn = hf == 0 ? fmin0 : fmin1, fmx = hf == 0 ? fmax0 : fmax1;
    uint32_t kmin = fmn <= fmx ? dsa::order_key(fmn) : 0xFFFFFFFFu;
    uint32_t kmax = fmn <= fmx ? dsa::order_key(fmx) : 0u;
    kmin = dsa::wave_min_u32(kmin);
    kmax = dsa::wave_max_u32(kmax);
    if (lane == 0) { red[(2 * hf) * kWaves + wave] = kmin; red[(2 * hf + 1) * kWaves + wave] = kmax; }
  }
  dsa::lds_barrier();
  if (threadIdx.x < kHalves && blk_minmax) {
    const int hf = threadIdx.x;
    if (kb + hf * kScoreBlock < n) {
      uint32_t mn = red[(2 * hf) * kWaves], mx = red[(2 * hf + 1) * kWaves];
      for (int i = 1; i < kWaves; ++i) {
        mn = min(mn, red[(2 * hf) * kWaves + i]);
        mx = max(mx, red[(2 * hf + 1) * kWaves + i]);
      }
      const int64_t e = int64_t(t) * nb_max + int64_t(blockIdx.x) * kHalves + hf;
      blk_minmax[2 * e] = mn;
      blk_minmax[2 * e + 1] = mx;
    }
  }
  if constexpr (MODE == kHist) {
    // The block's keys on fixed bins (order key >> 16) over a window of at most kWin bins ending at
    // the block's highest: suffix counts for the select, and the block's top keys, highest bins
    // first, down to the bin c where the block reaches its list length (ScoreHist).
    constexpr int kWin = ScoreHist::kWin;
    constexpr int kT = kWaves * 64;
    constexpr int kPer = KPB / kT;                        // keys per thread
    static_assert((2 * kWin + 1 + kT) * 4 <= int(sizeof(ring)), "counts and cursors fit in the ring");
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
    for (int i = 0; i < kHalves * kWaves; ++i) {
      kmn = min(kmn, red[2 * (i / kWaves) * kWaves + i % kWaves]);
      kmx = max(kmx, red[(2 * (i / kWaves) + 1) * kWaves + i % kWaves]);
    }
    const uint32_t hb = kmx >> 16, lb0 = kmn >> 16;
    const uint32_t lb = hb - lb0 >= uint32_t(kWin) ? hb - uint32_t(kWin - 1) : lb0;
    // hl: counts, then keys in bins >= each entry (hl[kWin] stays 0); cur: per-entry list cursors
    uint32_t* hl = reinterpret_cast<uint32_t*>(ring);   // the ring (or the staged queries) is free
    uint32_t* cur = hl + kWin + 1;
    for (int i = threadIdx.x; i <= 2 * kWin; i += kT) hl[i] = 0u;
    if (threadIdx.x == 0) s_c = 0u;
    dsa::lds_barrier();
    // Keys below the window (often half the block) all land in entry 0: they are counted by wave
    // ballots instead of atomics on that one address.
    // Every read first (no branch between them, so they are all in flight at once), then the
    // counts.
    uint32_t kk[kPer], ent[kPer];                         // order keys; entries (kWin: no key)
#pragma unroll
    for (int i = 0; i < kPer; ++i) kk[i] = dsa::order_key(s_sc[threadIdx.x + kT * i]);
    uint32_t n_low = 0u;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const bool valid = kb + int(threadIdx.x) + kT * i < kend;
      const uint32_t b = kk[i] >> 16;
      ent[i] = valid ? (b > lb ? b - lb : 0u) : uint32_t(kWin);
      const bool low = ent[i] == 0u;
      if (valid && !low) atomicAdd(&hl[ent[i]], 1u);
      n_low += uint32_t(__popcll(__builtin_amdgcn_ballot_w64(low)));
    }
    if (lane == 0 && n_low) atomicAdd(&hl[0], n_low);
    dsa::lds_barrier();
    // counts -> keys in bins >= lb + e, in place: thread k takes entries kWin-1-kPerT*k .. downward
    constexpr int kPerT = kWin / kT;
    static_assert(kPerT * kT == kWin, "whole entries per thread");
    uint32_t part[kPerT];
    uint32_t run = 0u;
#pragma unroll
    for (int i = 0; i < kPerT; ++i) {
      run += hl[kWin - 1 - (kPerT * threadIdx.x + i)];
      part[i] = run;
    }
    uint32_t incl = dsa::wave_incl_sum_u32(run);
    if (lane == 63) s_wsum[wave] = incl;
    dsa::lds_barrier();
    for (int w = 0; w < wave; ++w) incl += s_wsum[w];
    const uint32_t excl = incl - run;
    // the block's kWin counts side by side (entries past the block's highest bin hold 0): the
    // thread's kPerT entries are adjacent, so they go out as one store
    uint16_t* dst = hist.counts + (int64_t(t) * hist.g_max + blockIdx.x) * kWin + (kWin - kPerT * (threadIdx.x + 1));
    static_assert(kPerT == 4 || kPerT == 2, "a thread's counts fill one 8- or 4-byte store");
    uint32_t word[kPerT / 2];
#pragma unroll
    for (int i = 0; i < kPerT; ++i) {
      const int e = kWin - 1 - (kPerT * threadIdx.x + i);
      hl[e] = excl + part[i];
    }
    // entry kWin - kPerT * (k + 1) + m of thread k is its part[kPerT - 1 - m]
#pragma unroll
    for (int m = 0; m < kPerT / 2; ++m)
      word[m] = ((excl + part[kPerT - 1 - 2 * m]) & 0xFFFFu) | ((excl + part[kPerT - 2 - 2 * m]) << 16);
    if constexpr (kPerT == 4)
      *reinterpret_cast<uint2*>(dst) = make_uint2(word[0], word[1]);
    else
      *reinterpret_cast<uint32_t*>(dst) = word[0];
    dsa::lds_barrier();
    // c: the entry where the count from the top first reaches the list length (0 when it never
    // does: every key is listed)
    const uint32_t len = uint32_t(hist.list_len(n));
    {
      // the thread's entries and the one above them (hl[kWin] = 0)
      uint32_t v[kPerT + 1];
#pragma unroll
      for (int i = 0; i <= kPerT; ++i) v[i] = hl[kWin - kPerT * threadIdx.x - i];
#pragma unroll
      for (int i = 1; i <= kPerT; ++i)
        if (v[i] >= len && v[i - 1] < len) s_c = uint32_t(kWin - kPerT * threadIdx.x - i);
    }
    dsa::lds_barrier();
    const uint32_t c = s_c;
    // the keys of entries >= c, each at (keys in higher bins) + its place in its bin; places in
    // entry 0 (listed only when the whole block is) are handed out a wave at a time
    uint64_t* lst = hist.lists + (int64_t(t) * hist.g_max + blockIdx.x) * KPB;
    // the start of every key's entry (unconditional reads, all in flight), then the places
    uint32_t at[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) at[i] = hl[ent[i] < uint32_t(kWin) ? ent[i] + 1 : kWin];
    // Every lane takes part in every place atomic, so that no result waits inside a branch: a
    // key that is not listed (or sits in entry 0) adds 0 at a slot of its own thread.
    uint32_t* own = cur + kWin;                           // one dummy slot per thread
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const bool take = ent[i] < uint32_t(kWin) && ent[i] >= c && ent[i] != 0u;
      const uint32_t r = atomicAdd(take ? &cur[ent[i]] : &own[threadIdx.x], take ? 1u : 0u);
      at[i] += take ? r : 0u;
    }
    if (c == 0u) {
      // entry 0 is listed (the whole block is): its places go out a wave at a time
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const bool zero = ent[i] == 0u;
        const uint64_t m = __builtin_amdgcn_ballot_w64(zero);
        if (m) {
          const int first = __builtin_ctzll(m);
          uint32_t base = 0u;
          if (lane == first) base = atomicAdd(&cur[0], uint32_t(__popcll(m)));
          base = uint32_t(__builtin_amdgcn_readlane(int(base), first));
          if (zero)
            at[i] += base + uint32_t(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32),
                                                                __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (ent[i] < uint32_t(kWin) && ent[i] >= c)
        lst[at[i]] = (uint64_t(kk[i]) << 32) | uint32_t(~uint32_t(kb + int(threadIdx.x) + kT * i));
    }
    if (threadIdx.x == 0)
      hist.range[int64_t(t) * hist.g_max + blockIdx.x] =
          make_uint4(lb | (lb0 < lb ? 0x80000000u : 0u), hb, hl[c], 0u);
  }
}

}  // namespace

bool index_mfma_supported(const dsa_config& c) {
  const bool pow2 = c.page_size > 0 && (c.page_size & (c.page_size - 1)) == 0;
  return c.n_index_heads == H && c.index_dim == D && c.index_q_fmt == DSA_FMT_BF16 &&
         (c.index_key_fmt == DSA_FMT_BF16 || c.index_key_fmt == DSA_FMT_FP8) && pow2;
}

hipError_t launch_index_scores_mfma(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                                    const RowMap& map, const void* q, const float* w,
                                    const void* pool, float* scores, int64_t ld, bool fill,
                                    uint32_t* blk_minmax, int nb_max, uint32_t* run_max,
                                    int64_t rm_ld, const ScoreHist* hist, hipStream_t st) {
  const int n_rows = map.first[map.n];
  if (n_rows == 0) return hipSuccess;
  const dsa_config& c = h->cfg;
  int log2_ps = 0;
  while ((1 << log2_ps) < c.page_size) ++log2_ps;
  const int64_t cols = fill ? ld : in.max_visible;
  dim3 grid(unsigned((cols + KPB - 1) / KPB), unsigned(n_rows));
  // the block's page ids: at most KPB / page_size + 2 pages (a block need not start on a page)
  const size_t pages_bytes = size_t((KPB / c.page_size + 2 + 3) / 4 * 4) * 4 + (hist ? KPB * 4 : 0);
  const bool off32 = int64_t(p.pool_pages) * h->index_page_bytes <= int64_t(0xFFFFFFFFu);
  const ScoreHist hs = hist ? *hist : ScoreHist{};
#define DSA_LAUNCH_R(K, O, M)                                                                     \
  hipLaunchKernelGGL((index_scores_mfma<K, O, M>), grid, dim3(kWaves * 64), pages_bytes, st, p, map, \
                     static_cast<const uint16_t*>(q), w, static_cast<const uint8_t*>(pool), scores, \
                     ld, h->index_page_bytes, log2_ps, blk_minmax, nb_max, fill ? 1 : 0, run_max, \
                     rm_ld, hs)
#define DSA_LAUNCH(K, O)                                           \
  do {                                                             \
    if (run_max) DSA_LAUNCH_R(K, O, kRuns);                        \
    else if (hist) DSA_LAUNCH_R(K, O, kHist);                      \
    else DSA_LAUNCH_R(K, O, kPlain);                               \
  } while (0)
  if (c.index_key_fmt == DSA_FMT_BF16) {
    if (off32) DSA_LAUNCH(DSA_FMT_BF16, true); else DSA_LAUNCH(DSA_FMT_BF16, false);
  } else {
    if (off32) DSA_LAUNCH(DSA_FMT_FP8, true); else DSA_LAUNCH(DSA_FMT_FP8, false);
  }
#undef DSA_LAUNCH
#undef DSA_LAUNCH_R
  return hipGetLastError();
}
