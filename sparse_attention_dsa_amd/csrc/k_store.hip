// store_keys: scatter this step's index keys into the paged index-key pool.
// Row t of span s goes to request-local position ctx_start + t - q_start (DSA resource page,
// store_keys; IndexKeyStore.append). Pure data movement: 8-byte vector copies, one wave per row.
#include "dsa_internal.hpp"

namespace {

__global__ void __launch_bounds__(64) store_keys_kernel(DevPlan p, const uint8_t* __restrict__ keys,
                                                        const float* __restrict__ scales,
                                                        uint8_t* __restrict__ pool, int row_bytes,
                                                        int64_t page_bytes, int scale_base, int fp8) {
  const int t = blockIdx.x;
  dsa_span sp;
  dsa::row_span(p.spans, p.n_spans, t, &sp);
  const int pos = sp.ctx_start + (t - sp.q_start);
  int off;
  const int page = dsa::page_of(p, sp, pos, &off);
  uint8_t* dst_page = pool + int64_t(page) * page_bytes;
  const uint64_t* src = reinterpret_cast<const uint64_t*>(keys + int64_t(t) * row_bytes);
  uint64_t* dst = reinterpret_cast<uint64_t*>(dst_page + int64_t(off) * row_bytes);
  for (int i = threadIdx.x; i < row_bytes / 8; i += 64) dst[i] = src[i];
  if (fp8 && threadIdx.x == 0)
    reinterpret_cast<float*>(dst_page + scale_base)[off] = scales[t];
}

}  // namespace

hipError_t launch_store_keys(const dsa_handle* h, const DevPlan& p, const void* keys,
                             const float* scales, void* key_pool, hipStream_t st) {
  const dsa_config& c = h->cfg;
  const bool fp8 = c.index_key_fmt == DSA_FMT_FP8;
  const int esize = c.index_key_fmt == DSA_FMT_F32 ? 4 : c.index_key_fmt == DSA_FMT_BF16 ? 2 : 1;
  const int row_bytes = c.index_dim * esize;
  hipLaunchKernelGGL(store_keys_kernel, dim3(p.n_rows), dim3(64), 0, st, p,
                     static_cast<const uint8_t*>(keys), scales, static_cast<uint8_t*>(key_pool),
                     row_bytes, h->index_page_bytes, c.page_size * c.index_dim, fp8 ? 1 : 0);
  return hipGetLastError();
}
