// Absorbed MLA over each row's picked latents on the matrix cores (DSA resource page: attend;
// ttnn.transformer.sparse_sdpa operation line): for row t and head h over picked positions j,
//   logit_j = sm_scale * (q_nope[h] . c_j[0:512] + q_pe[h] . c_j[512:576]),
//   out[h]  = sum_j softmax(logit)_j * c_j[0:512].
// Shapes: 512 + 64 latents (bf16 rows, or packed 656-byte fp8 rows), bf16 queries and output,
// heads a multiple of 64.
//
// A workgroup of 4 waves takes one row, 64 heads and one range of its picks (a split). Wave
// (hg, ch) owns 32 heads (hg) and, for P.V, output columns [256*ch, 256*ch + 256). Picks are
// processed in chunks of 32: their latent rows are gathered into one row-major bf16 LDS tile
// (fp8 codes are converted exactly; their 128-element group scales are kept apart). Then
//   Q.K^T  v_mfma_f32_16x16x32_bf16, A = latent rows (row-major LDS reads), B = the wave's
//          queries held in VGPRs; wave ch computes keys [16*ch, 16*ch+16) of the chunk;
//          fp8 rows accumulate each 128-dim group apart and scale it in fp32 (exact);
//   softmax online, in base 2, the running max raised only when a chunk exceeds it by more than
//          2^8 (the rescale of O is skipped otherwise; the result is unchanged);
//   P.V    v_mfma_f32_32x32x16_bf16, A = P (bf16, via LDS, scaled by the fp8 group scale),
//          B = latent columns read transposed from the same LDS tile with ds_read_b64_tr_b16.
// With one split the workgroup writes the bf16 output; with several it writes fp32 partials
// (max, sum, unnormalised O) that a combine kernel merges.
#include "dsa_internal.hpp"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int R = 512, PR = 64, KD = R + PR;   // latent, rope, qk width
constexpr int CH = 32;                         // picks per chunk
constexpr int LP = KD + 16;                    // LDS pitch of a latent row (bf16 elements)
constexpr int PP = CH + 8;                     // LDS pitch of a P row (bf16 elements)
constexpr int HPB = 64;                        // heads per workgroup
constexpr int kThreads = 256;
constexpr int kMaxPicks = 4096;                // picks per workgroup (token list in LDS)
constexpr float kLazy = 8.0f;                  // log2 headroom before O is rescaled

template <int LFMT> struct Fmt;
template <> struct Fmt<DSA_FMT_BF16> { static constexpr int kPieces = KD * 2 / 16; static constexpr int kRowBytes = KD * 2; };
template <> struct Fmt<DSA_FMT_FP8> { static constexpr int kPieces = (R + 16 + PR * 2) / 16; static constexpr int kRowBytes = R + 16 + PR * 2; };

struct Smem {
  uint16_t lat[CH * LP];            // latent rows of the chunk, bf16
  float gscale[CH][4];              // fp8 group scales of the chunk's rows
  uint16_t pbuf[2][4][32 * PP];     // P per head group and column group, [head][key]
  float mx[2][2][32];               // per (head group, key half) chunk max
  float alpha[2][32];               // per head group rescale factor of this chunk
  float lsum[2][2][32];             // per (head group, key half) final partial sums
  int tok[kMaxPicks];               // pool token index of each pick (-1 = none)
};

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

template <int LFMT>
__global__ void __launch_bounds__(kThreads, 1)
attend_mfma(DevPlan p, const int32_t* __restrict__ sel, const uint16_t* __restrict__ q_nope,
            const uint16_t* __restrict__ q_pe, const uint8_t* __restrict__ pool, float scale_log2,
            uint16_t* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_ml,
            int topk, int H, int n_splits, int log2_ps) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  constexpr int PPK = Fmt<LFMT>::kPieces;
  constexpr int RB = Fmt<LFMT>::kRowBytes;

  const int t = blockIdx.x;
  const int hbase = blockIdx.y * HPB;
  const int split = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hg = wave >> 1, ch = wave & 1;
  const int s_idx = dsa::find_span(p.spans, p.n_spans, t);
  const dsa_span sp = p.spans[s_idx];
  const int pos = sp.ctx_start + (t - sp.q_start);

  // this split's picks
  const int per = (topk + n_splits - 1) / n_splits;
  const int k0 = split * per, k1 = min(topk, k0 + per);
  const int npk = max(0, k1 - k0);
  for (int i = threadIdx.x; i < npk; i += kThreads) {
    const int j = sel[int64_t(t) * topk + k0 + i];
    int tok = -1;
    if (j >= 0 && j <= pos) {
      int off;
      const int pg = dsa::page_of(p, sp, j, &off);
      tok = (pg << log2_ps) + off;
    }
    sm.tok[i] = tok;
  }

  // queries of this wave's 32 heads as the B operand of Q.K^T: head 16*nt + col, dims 32*ks + 8*grp
  const int grp = lane >> 4, col = lane & 15;
  bf16x8 qb[2][18];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int h = hbase + hg * 32 + nt * 16 + col;
    const uint16_t* qn = q_nope + (int64_t(t) * H + h) * R;
    const uint16_t* qp = q_pe + (int64_t(t) * H + h) * PR;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qb[nt][ks] = *reinterpret_cast<const bf16x8*>(qn + 32 * ks + 8 * grp);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qb[nt][16 + ks] = *reinterpret_cast<const bf16x8*>(qp + 32 * ks + 8 * grp);
  }

  f32x16 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[i][v] = 0.0f;
  float m_run[2] = {-__builtin_inff(), -__builtin_inff()};   // per head 16*nt + col (log2 units)
  float l_run[2] = {0.0f, 0.0f};                             // this lane's partial sums
  __syncthreads();

  // gather registers for one chunk
  constexpr int kLoads = (CH * PPK + kThreads - 1) / kThreads;
  u32x4 gr[kLoads];
  auto gather = [&](int c0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int piece = threadIdx.x + i * kThreads;
      gr[i] = u32x4{0u, 0u, 0u, 0u};
      if (piece < CH * PPK) {
        const int k = piece / PPK, pk = piece % PPK;
        const int idx = c0 + k;
        const int tok = idx < npk ? sm.tok[idx] : -1;
        if (tok >= 0)
          gr[i] = *reinterpret_cast<const u32x4*>(pool + int64_t(tok) * RB + 16 * pk);
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int piece = threadIdx.x + i * kThreads;
      if (piece >= CH * PPK) continue;
      const int k = piece / PPK, pk = piece % PPK;
      uint16_t* row = sm.lat + k * LP;
      if constexpr (LFMT == DSA_FMT_BF16) {
        *reinterpret_cast<u32x4*>(row + 8 * pk) = gr[i];
      } else {
        if (pk < 32) {
          u32x4 lo, hi;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(gr[i][d], 1.0f, false);
            const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(gr[i][d], 1.0f, true);
            const uint32_t wa = __builtin_bit_cast(uint32_t, a), wb = __builtin_bit_cast(uint32_t, b);
            if (d < 2) { lo[2 * d] = wa; lo[2 * d + 1] = wb; } else { hi[2 * (d - 2)] = wa; hi[2 * (d - 2) + 1] = wb; }
          }
          *reinterpret_cast<u32x4*>(row + 16 * pk) = lo;
          *reinterpret_cast<u32x4*>(row + 16 * pk + 8) = hi;
        } else if (pk == 32) {
          sm.gscale[k][0] = __uint_as_float(gr[i][0]);
          sm.gscale[k][1] = __uint_as_float(gr[i][1]);
          sm.gscale[k][2] = __uint_as_float(gr[i][2]);
          sm.gscale[k][3] = __uint_as_float(gr[i][3]);
        } else {
          *reinterpret_cast<u32x4*>(row + R + 8 * (pk - 33)) = gr[i];
        }
      }
    }
  };

  const int n_chunks = (npk + CH - 1) / CH;
  if (n_chunks > 0) gather(0);
  for (int c = 0; c < n_chunks; ++c) {
    __syncthreads();                       // previous chunk's LDS reads are done
    stage();
    __syncthreads();                       // chunk tile ready
    if (c + 1 < n_chunks) gather((c + 1) * CH);

    // ---- Q.K^T for keys [16*ch, 16*ch + 16) of the chunk, 32 heads
    f32x4 acc[2][5];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int g = 0; g < 5; ++g) acc[nt][g] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* arow = sm.lat + (16 * ch + col) * LP + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + 32 * ks);
      const int g = LFMT == DSA_FMT_FP8 ? (ks < 16 ? ks / 4 : 4) : 0;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        acc[nt][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[nt][ks], acc[nt][g], 0, 0, 0);
    }
    // logits (log2 units) of keys 16*ch + 4*grp + v for head 16*nt + col
    float lg[2][4];
    bool valid[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int idx = c * CH + 16 * ch + 4 * grp + v;
      valid[v] = idx < npk && sm.tok[idx] >= 0;
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float x;
        if constexpr (LFMT == DSA_FMT_FP8) {
          const float* gs = sm.gscale[16 * ch + 4 * grp + v];
          x = acc[nt][4][v];
          x = fmaf(gs[0], acc[nt][0][v], x);
          x = fmaf(gs[1], acc[nt][1][v], x);
          x = fmaf(gs[2], acc[nt][2][v], x);
          x = fmaf(gs[3], acc[nt][3][v], x);
        } else {
          x = acc[nt][0][v];
        }
        lg[nt][v] = valid[v] ? x * scale_log2 : -__builtin_inff();
      }
    // this wave's max per head over its 16 keys
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float m = fmaxf(fmaxf(lg[nt][0], lg[nt][1]), fmaxf(lg[nt][2], lg[nt][3]));
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      if (grp == 0) sm.mx[hg][ch][nt * 16 + col] = m;
    }
    __syncthreads();
    float pv[2][4];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float mc = fmaxf(sm.mx[hg][0][nt * 16 + col], sm.mx[hg][1][nt * 16 + col]);
      float alpha = 1.0f;
      if (mc > m_run[nt] + kLazy) {          // raise the running max; O and sums rescale
        alpha = exp2f(m_run[nt] - mc);       // 0 when nothing was accumulated yet
        m_run[nt] = mc;
        l_run[nt] *= alpha;
      }
      if (ch == 0 && grp == 0) sm.alpha[hg][nt * 16 + col] = alpha;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        pv[nt][v] = valid[v] ? exp2f(lg[nt][v] - m_run[nt]) : 0.0f;
        l_run[nt] += pv[nt][v];
      }
      // P[head][key] for every column group this chunk's consumers need
      const int head = nt * 16 + col;
      const int kk = 16 * ch + 4 * grp;
      constexpr int NG = LFMT == DSA_FMT_FP8 ? 4 : 1;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        float s0 = 1.f, s1 = 1.f, s2 = 1.f, s3 = 1.f;
        if constexpr (LFMT == DSA_FMT_FP8) {
          s0 = sm.gscale[kk][g]; s1 = sm.gscale[kk + 1][g]; s2 = sm.gscale[kk + 2][g]; s3 = sm.gscale[kk + 3][g];
        }
        bf16x4 pk4;
        pk4[0] = (__bf16)(pv[nt][0] * s0);
        pk4[1] = (__bf16)(pv[nt][1] * s1);
        pk4[2] = (__bf16)(pv[nt][2] * s2);
        pk4[3] = (__bf16)(pv[nt][3] * s3);
        *reinterpret_cast<bf16x4*>(sm.pbuf[hg][g] + head * PP + kk) = pk4;
      }
    }
    __syncthreads();

    // ---- rescale O where the running max moved (rare)
    {
      // O layout: lane holds heads 8*(v/4) + 4*(lane/32) + v%4, column lane%32
      bool any = false;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int r = 0; r < 4; ++r) any |= sm.alpha[hg][8 * q4 + 4 * (lane >> 5) + r] != 1.0f;
      if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float a = sm.alpha[hg][8 * (v / 4) + 4 * (lane >> 5) + (v % 4)];
#pragma unroll
          for (int i = 0; i < 8; ++i) o[i][v] *= a;
        }
      }
    }

    // ---- P.V: 32 heads x 256 columns, keys of the whole chunk (2 k-steps of 16)
    const int half = lane >> 5;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8 pa[LFMT == DSA_FMT_FP8 ? 2 : 1];
#pragma unroll
      for (int gi = 0; gi < (LFMT == DSA_FMT_FP8 ? 2 : 1); ++gi) {
        const int g = LFMT == DSA_FMT_FP8 ? 2 * ch + gi : 0;
        pa[gi] = *reinterpret_cast<const bf16x8*>(sm.pbuf[hg][g] + (lane & 31) * PP + 16 * u + 8 * half);
      }
      // transposed reads: source lane (4r + q) of each 16-lane group points at row
      // 16u + 8*half + r (+4), columns 16*cb + 4q of the tile
      const int li = lane & 15, r = li >> 2, q = li & 3, cb = (lane >> 4) & 1;
      const uint16_t* vbase = sm.lat + (16 * u + 8 * half + r) * LP + 256 * ch + 16 * cb + 4 * q;
#pragma unroll
      for (int nt2 = 0; nt2 < 8; ++nt2) {
        const uint16_t* va = vbase + 32 * nt2;
        // whole-vector shuffle: an element-wise bit cast of shorts into the operand is miscompiled
        const bf16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (bf16x4 __attribute__((address_space(3)))*)(va));
        const bf16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (bf16x4 __attribute__((address_space(3)))*)(va + 4 * LP));
        const bf16x8 b = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
        const int gi = LFMT == DSA_FMT_FP8 ? (nt2 >> 2) : 0;
        o[nt2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[gi], b, o[nt2], 0, 0, 0);
      }
    }
  }

  // ---- row sums: reduce this lane's partials over the 4 lane groups, then the key halves
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float s = l_run[nt];
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if (grp == 0) {
      sm.lsum[hg][ch][nt * 16 + col] = s;
      if (ch == 0) sm.mx[hg][0][nt * 16 + col] = m_run[nt];
    }
  }
  __syncthreads();
  const int half = lane >> 5;
  const int64_t orow = int64_t(t) * H + hbase + hg * 32;
  if (n_splits == 1) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int head = 8 * (v / 4) + 4 * half + (v % 4);
      const float l = sm.lsum[hg][0][head] + sm.lsum[hg][1][head];
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
      uint16_t* dst = out + (orow + head) * R + 256 * ch + (lane & 31);
#pragma unroll
      for (int nt2 = 0; nt2 < 8; ++nt2) dst[32 * nt2] = dsa::f32_to_bf16(o[nt2][v] * inv);
    }
  } else {
    const int64_t prow = (int64_t(t) * n_splits + split) * H + hbase + hg * 32;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int head = 8 * (v / 4) + 4 * half + (v % 4);
      float* dst = part_o + (prow + head) * R + 256 * ch + (lane & 31);
#pragma unroll
      for (int nt2 = 0; nt2 < 8; ++nt2) dst[32 * nt2] = o[nt2][v];
    }
    if (ch == 0 && lane < 32) {
      const int head = lane;
      part_ml[2 * (prow + head)] = sm.mx[hg][0][head];
      part_ml[2 * (prow + head) + 1] = sm.lsum[hg][0][head] + sm.lsum[hg][1][head];
    }
  }
}

// out[t][h] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the splits.
__global__ void __launch_bounds__(256)
attend_combine(const float* __restrict__ part_o, const float* __restrict__ part_ml,
               uint16_t* __restrict__ out, int H, int n_splits) {
  const int t = blockIdx.x, h = blockIdx.y;
  float M = -__builtin_inff();
  for (int s = 0; s < n_splits; ++s) M = fmaxf(M, part_ml[2 * ((int64_t(t) * n_splits + s) * H + h)]);
  float wsum = 0.0f;
  float acc[2] = {0.0f, 0.0f};
  for (int s = 0; s < n_splits; ++s) {
    const int64_t row = (int64_t(t) * n_splits + s) * H + h;
    const float m = part_ml[2 * row], l = part_ml[2 * row + 1];
    if (!(l > 0.0f)) continue;
    const float wgt = exp2f(m - M);
    wsum += wgt * l;
    acc[0] += wgt * part_o[row * R + threadIdx.x];
    acc[1] += wgt * part_o[row * R + 256 + threadIdx.x];
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  uint16_t* dst = out + (int64_t(t) * H + h) * R;
  dst[threadIdx.x] = dsa::f32_to_bf16(acc[0] * inv);
  dst[256 + threadIdx.x] = dsa::f32_to_bf16(acc[1] * inv);
}

int pick_splits(const PlanInfo& in, int H, int topk) {
  // enough workgroups to cover the chip (256 CUs, one workgroup each), at least 64 picks each
  const int base = in.n_rows * (H / HPB);
  int s = 1;
  while (base * s < 256 && s * 2 * 64 <= topk && s < 32) s *= 2;
  return s;
}

}  // namespace

bool attend_mfma_supported(const dsa_config& c) {
  const bool pow2 = c.page_size > 0 && (c.page_size & (c.page_size - 1)) == 0;
  return c.q_fmt == DSA_FMT_BF16 && (c.latent_fmt == DSA_FMT_BF16 || c.latent_fmt == DSA_FMT_FP8) &&
         c.kv_lora_rank == R && c.rope_dim == PR && c.n_heads % HPB == 0 && c.topk <= kMaxPicks && pow2;
}

size_t attend_mfma_workspace(const dsa_config& c, const PlanInfo& in) {
  const int s = pick_splits(in, c.n_heads, c.topk);
  if (s == 1) return 0;
  const size_t rows = size_t(in.n_rows) * s * c.n_heads;
  return ((rows * R * 4 + 255) & ~size_t(255)) + rows * 8;
}

hipError_t launch_attend_mfma(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                              const int32_t* sel, const void* qn, const void* qp, const void* pool,
                              float sm_scale, void* out, void* ws, hipStream_t st) {
  const dsa_config& c = h->cfg;
  const int s = pick_splits(in, c.n_heads, c.topk);
  int log2_ps = 0;
  while ((1 << log2_ps) < c.page_size) ++log2_ps;
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (s > 1) {
    const size_t rows = size_t(in.n_rows) * s * c.n_heads;
    part_o = static_cast<float*>(ws);
    part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + ((rows * R * 4 + 255) & ~size_t(255)));
  }
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  dim3 grid(in.n_rows, c.n_heads / HPB, s);
  const size_t lds = sizeof(Smem);
  if (c.latent_fmt == DSA_FMT_BF16)
    hipLaunchKernelGGL(attend_mfma<DSA_FMT_BF16>, grid, dim3(kThreads), lds, st, p, sel,
                       static_cast<const uint16_t*>(qn), static_cast<const uint16_t*>(qp),
                       static_cast<const uint8_t*>(pool), scale_log2, static_cast<uint16_t*>(out),
                       part_o, part_ml, c.topk, c.n_heads, s, log2_ps);
  else
    hipLaunchKernelGGL(attend_mfma<DSA_FMT_FP8>, grid, dim3(kThreads), lds, st, p, sel,
                       static_cast<const uint16_t*>(qn), static_cast<const uint16_t*>(qp),
                       static_cast<const uint8_t*>(pool), scale_log2, static_cast<uint16_t*>(out),
                       part_o, part_ml, c.topk, c.n_heads, s, log2_ps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || s == 1) return e;
  hipLaunchKernelGGL(attend_combine, dim3(in.n_rows, c.n_heads), dim3(256), 0, st, part_o, part_ml,
                     static_cast<uint16_t*>(out), c.n_heads, s);
  return hipGetLastError();
}
