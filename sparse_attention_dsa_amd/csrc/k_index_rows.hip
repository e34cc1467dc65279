// Indexer score for requests with many rows in the step (prefill and chunked prefill), on the
// matrix cores, 64 heads x 128 dims, bf16 queries, bf16 or fp8 keys:
//   s[t][j] = sum_h w[t][h] * relu(q[t][h] . k_j),  j = 0 .. position(t)
// (DSA resource page: module description, index_topk.)
//
// A workgroup (4 waves) scores a group of 8 consecutive rows of one request against KPB
// consecutive keys of that request, so every key it loads serves 8 rows. Wave w owns rows 2w and
// 2w + 1: their 64 x 128 queries stay in VGPRs as the A operand of v_mfma_f32_16x16x32_bf16
// (heads are M, keys are N, dims are K). Keys go from HBM straight into an LDS ring of 64-key
// chunks with global_load_lds (16 bytes a lane, each instruction a contiguous 1 KB of whole key
// rows); the 16-byte pieces of a key's row are XOR-swizzled by the key index, which keeps the
// B-operand reads free of bank conflicts. Lane l takes key l%16 and the pieces l/16, l/16 + 4, ...
// of its row (fp8 codes become bf16 exactly in registers), and the A operand takes the query's
// dims in the same order, so the contraction is unchanged. The epilogue matches the single-row
// kernel's: relu, head weight, a lane sum over 16 heads and two lane swaps for all 64; an fp8
// key's scale (>= 0) multiplies the finished sum. Keys past a row's position score -inf. Each
// row's min and max order key over the block go to the top-k select.
//
// The launch runs group-major (blockIdx.x = group, blockIdx.y = key block), so the workgroups
// resident at one time read the same key block and it is served from L2. Within a chunk the
// work is software-pipelined: the MFMAs of one (tile, row) stage are interleaved with the relu
// and weighting of the stage before, and the reduction over lane quarters is done for the four
// tiles of a chunk at once.
#include "dsa_internal.hpp"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int H = 64, D = 128;
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 2;
static_assert(kWaves * kRowsPerWave == RowGroups::kRows, "one group per workgroup");
constexpr int KPB = kScoreBlock;          // keys per workgroup
constexpr int CK = 64;                    // keys per LDS chunk (4 tiles of 16)
constexpr int NB = 3;                     // chunks in the ring
constexpr int kStores = kRowsPerWave;   // score stores per wave per chunk

template <int KFMT> struct KT;
template <> struct KT<DSA_FMT_BF16> {
  static constexpr int kRow = 2 * D;      // bytes of a key
  static constexpr int kScaleBytes = 0;
};
template <> struct KT<DSA_FMT_FP8> {
  static constexpr int kRow = D;
  static constexpr int kScaleBytes = kWaves * 256;   // wave w: scales of keys 16w .. 16w+15
};

template <int KFMT> struct Smem {
  static constexpr int kChunk = CK * KT<KFMT>::kRow + KT<KFMT>::kScaleBytes;
  uint8_t ring[NB][kChunk];
  uint32_t pages[KPB + 2];                // page ids of the block's pages
};

__device__ __forceinline__ void dma16(const void* src, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

template <int KFMT>
__global__ void __launch_bounds__(kWaves * 64, 2)
index_scores_rows(DevPlan p, RowGroups groups, const uint16_t* __restrict__ q,
                  const float* __restrict__ w, const uint8_t* __restrict__ pool,
                  float* __restrict__ scores, int64_t ld, int64_t page_bytes, int log2_ps,
                  uint32_t* __restrict__ blk_minmax, int nb_max, int fill_masked) {
  constexpr bool FP8 = KFMT == DSA_FMT_FP8;
  constexpr int kRow = KT<KFMT>::kRow;
  constexpr int kPieces = kRow / 16;                       // 16-byte pieces of a key: 16 or 8
  constexpr int kInstr = CK * kPieces / 64 / kWaves;       // row DMAs per wave per chunk
  constexpr int kOps = kInstr + (FP8 ? 1 : 0);             // vector-memory ops per wave per chunk
  static_assert(NB == 3, "the wait counts below assume a ring of three chunks");
  __shared__ __attribute__((aligned(16))) Smem<KFMT> sm;

  // This workgroup's request, rows and key block. Workgroups go out in reverse order, last key
  // block and last group first: the small workgroups on the causal diagonal then come at the end
  // instead of leaving a tail of full-size ones.
  const int gid = groups.first[groups.n_spans] - 1 - int(blockIdx.x);
  const int blk = int(gridDim.y) - 1 - int(blockIdx.y);
  int gs = 0;
  while (gs + 1 < groups.n_spans && groups.first[gs + 1] <= gid) ++gs;
  const dsa_span sp = p.spans[groups.span[gs]];
  const int t0 = sp.q_start + RowGroups::kRows * (gid - groups.first[gs]);
  const int pos0 = sp.ctx_start + (t0 - sp.q_start);        // position of row t0
  const int pmax = pos0 + RowGroups::kRows - 1;
  const int kb = blk * KPB;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4, col = lane & 15;

  if (kb > pmax) {
    if (fill_masked)
      for (int r = 0; r < RowGroups::kRows; ++r)
        for (int j = kb + threadIdx.x; j < ld && j < kb + KPB; j += kWaves * 64)
          scores[int64_t(t0 + r) * ld + j] = -__builtin_inff();
    return;
  }
  const int kend = min(pmax + 1, kb + KPB);                // keys any row of the group needs
  const int first_list = (sp.page_start + kb) >> log2_ps;
  const int last_list = (sp.page_start + kend - 1) >> log2_ps;
  for (int i = threadIdx.x; i <= last_list - first_list; i += kWaves * 64) {
    const int pg = p.page_table[dsa::page_entry(sp, first_list + i)];
    sm.pages[i] = uint32_t(pg < 0 ? 0 : (pg >= p.pool_pages ? p.pool_pages - 1 : pg));
  }

  // this wave's rows: A operands (head 16*mt + col, the dims of k-step ks in the B fragment's
  // order) and the head weights of the accumulator rows the lane holds (head 16*mt + 4*grp + v)
  int rows[kRowsPerWave], rpos[kRowsPerWave];
  bf16x8 a[kRowsPerWave][4][4];
  float wr[kRowsPerWave][16];
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int r = kRowsPerWave * wave + rr;
    rows[rr] = t0 + r;
    rpos[rr] = pos0 + r;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int d0 = FP8 ? 64 * (ks >> 1) + 16 * grp + 8 * (ks & 1) : 32 * ks + 8 * grp;
        a[rr][mt][ks] = *reinterpret_cast<const bf16x8*>(q + (int64_t(rows[rr]) * H + 16 * mt + col) * D + d0);
      }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) wr[rr][mt * 4 + v] = w[int64_t(rows[rr]) * H + 16 * mt + 4 * grp + v];
  }
  // Pin the operands here so that their loads are complete before the ring starts: from now on
  // the vector-memory counter holds only this wave's DMAs and score stores, which the waits count.
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(wr[rr][i]));
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) asm volatile("" : "+v"(a[rr][mt][ks]));
  }
  wait_vmcnt<0>();
  __syncthreads();                                          // page ids staged

  const uint32_t ring0 = lds_u32(&sm.ring[0][0]);
  const int n_chunks = (kend - kb + CK - 1) / CK;
  // DMA of chunk c into ring slot r, this wave's share. Instruction m fills the chunk's 16-byte
  // cells 64m .. 64m + 63; cell s holds piece (s % P) ^ (k % P) of key k = s / P (P pieces a
  // key). Keys past kend load key kend - 1, whose scores are never kept.
  // Addresses first, then the DMAs: the page-id reads then overlap instead of each waiting
  // behind the previous DMA.
  auto issue = [&](int c, int r) {
    const int key0 = kb + c * CK;
    const uint8_t* src[kOps];
#pragma unroll
    for (int i = 0; i < kInstr; ++i) {
      const int s = 64 * (wave * kInstr + i) + lane;
      const int k = s / kPieces;
      const int pc = (s % kPieces) ^ (k % kPieces);
      const int slot = sp.page_start + min(key0 + k, kend - 1);
      const uint32_t pg = sm.pages[(slot >> log2_ps) - first_list];
      const uint32_t off = uint32_t(slot & ((1 << log2_ps) - 1));
      src[i] = pool + int64_t(pg) * page_bytes + off * uint32_t(kRow) + 16 * pc;
    }
    if constexpr (FP8) {
      // the page's scales follow its codes, 4 bytes a key
      const int slot = sp.page_start + min(key0 + 16 * wave + (lane & 15), kend - 1);
      const uint32_t pg = sm.pages[(slot >> log2_ps) - first_list];
      const uint32_t off = uint32_t(slot & ((1 << log2_ps) - 1));
      src[kInstr] = pool + int64_t(pg) * page_bytes + (uint32_t(1) << log2_ps) * D + off * 4;
    }
#pragma unroll
    for (int i = 0; i < kInstr; ++i)
      dma16(src[i], ring0 + uint32_t(r * Smem<KFMT>::kChunk + 1024 * (wave * kInstr + i)));
    if constexpr (FP8) dma4(src[kInstr], ring0 + uint32_t(r * Smem<KFMT>::kChunk + CK * kRow + 256 * wave));
  };

  float fmn[kRowsPerWave], fmx[kRowsPerWave];
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr) { fmn[rr] = __builtin_inff(); fmx[rr] = -__builtin_inff(); }

  issue(0, 0);
  if (n_chunks > 1) issue(1, 1);

#pragma clang loop unroll(disable)
  for (int c = 0; c < n_chunks; ++c) {
    const int r = c % NB;
    // Chunk c has landed once no more than the later ops are outstanding: the stores of chunks
    // c-2 and c-1 and, if it exists, the DMA of chunk c+1 (issued in order after chunk c's).
    if (c + 1 < n_chunks) {
      if (c >= 2) wait_vmcnt<kOps + 2 * kStores>();
      else if (c == 1) wait_vmcnt<kOps + kStores>();
      else wait_vmcnt<kOps>();
    } else {
      if (c >= 2) wait_vmcnt<2 * kStores>();
      else if (c == 1) wait_vmcnt<kStores>();
      else wait_vmcnt<0>();
    }
    // Every wave's share of chunk c is in, and every wave is done with chunk c-1 (its LDS reads
    // fed the MFMAs of the last iteration), whose slot the next DMA refills. A bare s_barrier:
    // the workgroup fence of __syncthreads would also wait for the score stores.
    __builtin_amdgcn_s_barrier();
    if (c + 2 < n_chunks) issue(c + 2, (c + 2) % NB);
    const uint32_t chunk = ring0 + uint32_t(r * Smem<KFMT>::kChunk);
    // B fragments of key 16*tt + col: pieces grp + 4i of its row
    auto load_b = [&](int tt, bf16x8* b) {
      const int kc = 16 * tt + col;
      u32x4 raw[kPieces / 4];
#pragma unroll
      for (int i = 0; i < kPieces / 4; ++i) {
        const uint32_t at = chunk + uint32_t(kc * kRow + 16 * ((grp + 4 * i) ^ (kc % kPieces)));
        raw[i] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(uintptr_t(at));
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if constexpr (!FP8) {
          b[ks] = __builtin_bit_cast(bf16x8, raw[ks]);
        } else {
          const uint32_t lo = raw[ks >> 1][(ks & 1) * 2], hi = raw[ks >> 1][(ks & 1) * 2 + 1];
          const bf16x2 x0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
          const bf16x2 x1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
          const bf16x2 x2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
          const bf16x2 x3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
          const bf16x4 ab = __builtin_shufflevector(x0, x1, 0, 1, 2, 3);
          const bf16x4 cd = __builtin_shufflevector(x2, x3, 0, 1, 2, 3);
          b[ks] = __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      }
    };
    // part[rr][tt]: for key 16*tt + col, this lane's 16 heads of row rr, weighted and summed.
    // Software pipeline over the chunk's 8 (tile, row) stages: stage s runs the 16 MFMAs of
    // tile s/2, row s%2, while the VALU works through the relu and weights of stage s-1, and the
    // B fragments of the next tile are read during the second row of the current one.
    float part[kRowsPerWave][CK / 16];
    bf16x8 b[2][4];
    f32x4 accp[4];
    load_b(0, b[0]);
#pragma unroll
    for (int st = 0; st <= 2 * (CK / 16); ++st) {
      f32x4 accn[4];
      if (st < 2 * (CK / 16)) {
        const int tt = st >> 1, rr = st & 1;
        if (rr == 1 && tt + 1 < CK / 16) load_b(tt + 1, b[(tt + 1) & 1]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) accn[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
            accn[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rr][mt][ks], b[tt & 1][ks], accn[mt], 0, 0, 0);
      }
      if (st > 0) {
        const int tp = (st - 1) >> 1, rp = (st - 1) & 1;
        // relu and head weight, as two fma chains over heads 16*mt + 4*grp + v
        float c0 = wr[rp][0] * relu_bits(accp[0][0]);
        float c1 = wr[rp][8] * relu_bits(accp[2][0]);
#pragma unroll
        for (int e = 1; e < 8; ++e) {
          c0 = fmaf(wr[rp][e], relu_bits(accp[e >> 2][e & 3]), c0);
          c1 = fmaf(wr[rp][8 + e], relu_bits(accp[2 + (e >> 2)][e & 3]), c1);
        }
        part[rp][tp] = c0 + c1;
      }
      if (st < 2 * (CK / 16)) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) accp[mt] = accn[mt];
        // interleave: each MFMA followed by two VALU instructions of the previous stage
        if (st > 0) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
          }
        }
      }
    }
    // Lane l holds, per tile, one quarter of the heads (row l/16 of the accumulators) of key
    // 16*tt + l%16. Two rounds of lane-half swaps add the quarters and leave lane l with the whole
    // score of chunk key l: v_permlane32_swap puts tiles 0 and 2 (1 and 3) side by side with
    // their row pairs (0,2) and (1,3) added, v_permlane16_swap then adds rows 0+1 and 2+3 and
    // interleaves the tiles back into key order.
    const int j = min(kb + c * CK + lane, kend - 1);       // a lane past kend repeats key kend-1
    float scale = 1.0f;
    if constexpr (FP8) {
      const uint32_t at = chunk + uint32_t(CK * kRow + 256 * (lane >> 4) + 4 * (lane & 15));
      scale = *reinterpret_cast<const __attribute__((address_space(3))) float*>(uintptr_t(at));
    }
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
      const auto p02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[rr][0]), __float_as_uint(part[rr][2]), false, false);
      const auto p13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[rr][1]), __float_as_uint(part[rr][3]), false, false);
      const float x = __uint_as_float(p02[0]) + __uint_as_float(p02[1]);
      const float y = __uint_as_float(p13[0]) + __uint_as_float(p13[1]);
      const auto pxy = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
      const float val = (__uint_as_float(pxy[0]) + __uint_as_float(pxy[1])) * scale;
      const bool seen = j <= rpos[rr];                      // causal: key j is visible to the row
      // one store per row and chunk, every lane active, so the waits above count exactly
      scores[int64_t(rows[rr]) * ld + j] = seen ? val : -__builtin_inff();
      fmn[rr] = fminf(fmn[rr], seen ? val : __builtin_inff());
      fmx[rr] = fmaxf(fmx[rr], seen ? val : -__builtin_inff());
    }
  }

  // -inf past the block's last needed key (fill mode), per row; each row's min / max
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    if (fill_masked)
      for (int jj = kend + lane; jj < kb + KPB && jj < ld; jj += 64)
        scores[int64_t(rows[rr]) * ld + jj] = -__builtin_inff();
    uint32_t kmin = fmn[rr] <= fmx[rr] ? dsa::order_key(fmn[rr]) : 0xFFFFFFFFu;
    uint32_t kmax = fmn[rr] <= fmx[rr] ? dsa::order_key(fmx[rr]) : 0u;
    kmin = dsa::wave_min_u32(kmin);
    kmax = dsa::wave_max_u32(kmax);
    if (lane == 0 && blk_minmax && kb <= rpos[rr]) {
      blk_minmax[2 * (int64_t(rows[rr]) * nb_max + blk)] = kmin;
      blk_minmax[2 * (int64_t(rows[rr]) * nb_max + blk) + 1] = kmax;
    }
  }
}

}  // namespace

void split_rows(const PlanInfo& in, RowGroups* g, RowMap* m) {
  g->n_spans = 0;
  g->first[0] = 0;
  m->n = 0;
  m->first[0] = 0;
  int mapped = 0;        // rows in the map so far
  int run_end = -1;      // step row just past the map's last range
  auto add_rows = [&](int t, int count) {
    if (count <= 0) return;
    if (m->n > 0 && run_end == t) {
      m->first[m->n] += count;
    } else {
      m->start[m->n] = t;
      m->first[m->n + 1] = mapped + count;
      ++m->n;
    }
    mapped += count;
    run_end = t + count;
  };
  for (int s = 0; s < in.n_spans; ++s) {
    const dsa_span& sp = in.spans_host[s];
    int grouped = 0;
    if (sp.q_len >= RowGroups::kMinQLen && g->n_spans < RowGroups::kMaxSpans) {
      const int ng = sp.q_len / RowGroups::kRows;
      g->span[g->n_spans] = s;
      g->first[g->n_spans + 1] = g->first[g->n_spans] + ng;
      ++g->n_spans;
      grouped = ng * RowGroups::kRows;
    }
    add_rows(sp.q_start + grouped, sp.q_len - grouped);
  }
}

hipError_t launch_index_scores_rows(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                                    const RowGroups& g, const void* q, const float* w,
                                    const void* pool, float* scores, int64_t ld, bool fill,
                                    uint32_t* blk_minmax, int nb_max, hipStream_t st) {
  const int n_groups = g.first[g.n_spans];
  if (n_groups == 0) return hipSuccess;
  const dsa_config& c = h->cfg;
  int log2_ps = 0;
  while ((1 << log2_ps) < c.page_size) ++log2_ps;
  const int64_t cols = fill ? ld : in.max_visible;
  dim3 grid(unsigned(n_groups), unsigned((cols + KPB - 1) / KPB));
  if (c.index_key_fmt == DSA_FMT_BF16)
    hipLaunchKernelGGL(index_scores_rows<DSA_FMT_BF16>, grid, dim3(kWaves * 64), 0, st, p, g,
                       static_cast<const uint16_t*>(q), w, static_cast<const uint8_t*>(pool), scores,
                       ld, h->index_page_bytes, log2_ps, blk_minmax, nb_max, fill ? 1 : 0);
  else
    hipLaunchKernelGGL(index_scores_rows<DSA_FMT_FP8>, grid, dim3(kWaves * 64), 0, st, p, g,
                       static_cast<const uint16_t*>(q), w, static_cast<const uint8_t*>(pool), scores,
                       ld, h->index_page_bytes, log2_ps, blk_minmax, nb_max, fill ? 1 : 0);
  return hipGetLastError();
}
