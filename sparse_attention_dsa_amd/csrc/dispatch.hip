// Kernel choice per configuration and plan.
#include "dsa_internal.hpp"

hipError_t launch_index_scores_generic(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                                       const void* q, const float* w, const void* pool,
                                       float* scores, int64_t ld, bool fill, hipStream_t st);
bool index_mfma_supported(const dsa_config& c);
hipError_t launch_index_scores_mfma(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                                    const RowMap& map, const void* q, const float* w,
                                    const void* pool, float* scores, int64_t ld, bool fill,
                                    uint32_t* blk_minmax, int nb_max, uint32_t* run_max,
                                    int64_t rm_ld, const ScoreHist* hist, hipStream_t st);
hipError_t launch_index_scores_rows(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                                    const RowGroups& g, const void* q, const float* w,
                                    const void* pool, float* scores, int64_t ld, bool fill,
                                    uint32_t* blk_minmax, int nb_max, hipStream_t st);

// Matrix-core scores of every row: groups of rows of long spans share key tiles, the other rows
// are scored one per workgroup. The two launches write disjoint rows.
static hipError_t index_scores_mfma_all(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                                        const void* q, const float* w, const void* pool,
                                        float* scores, int64_t ld, bool fill, uint32_t* mm,
                                        int nb_max, hipStream_t st) {
  RowGroups g;
  RowMap map;
  split_rows(in, &g, &map);
  hipError_t e = launch_index_scores_rows(h, p, in, g, q, w, pool, scores, ld, fill, mm, nb_max, st);
  if (e != hipSuccess) return e;
  return launch_index_scores_mfma(h, p, in, map, q, w, pool, scores, ld, fill, mm, nb_max, nullptr,
                                  0, nullptr, st);
}
uint32_t* select_minmax_buffer(const dsa_handle* h, const PlanInfo& in, void* ws, int* nb_max);
hipError_t launch_select_topk_ex(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                                 const float* scores, int64_t ld, int32_t* sel, void* ws,
                                 bool have_minmax, hipStream_t st);
hipError_t launch_attend_generic(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                                 const int32_t* sel, const void* qn, const void* qp,
                                 const void* pool, float sm_scale, const float* sink, void* out,
                                 hipStream_t st);

hipError_t launch_index_scores(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                               const void* q, const float* w, const void* key_pool, float* scores,
                               int64_t ld, bool fill_masked, hipStream_t st) {
  if (index_mfma_supported(h->cfg))
    return index_scores_mfma_all(h, p, in, q, w, key_pool, scores, ld, fill_masked, nullptr, 0, st);
  return launch_index_scores_generic(h, p, in, q, w, key_pool, scores, ld, fill_masked, st);
}

bool index_run_max_supported(const dsa_handle* h, const PlanInfo& in) {
  return index_mfma_supported(h->cfg) && in.all_decode;   // every row on the one-row kernel
}

hipError_t launch_index_scores_run_max(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                                       const void* q, const float* w, const void* key_pool,
                                       float* scores, int64_t ld, uint32_t* run_max, int64_t rm_ld,
                                       hipStream_t st) {
  RowGroups g;
  RowMap map;
  split_rows(in, &g, &map);
  return launch_index_scores_mfma(h, p, in, map, q, w, key_pool, scores, ld, false, nullptr, 0,
                                  run_max, rm_ld, nullptr, st);
}

ScoreHist select_hist_buffers(const dsa_handle* h, const PlanInfo& in, void* ws);
hipError_t launch_select_lists(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                               const float* scores, int64_t ld, int32_t* sel, void* ws,
                               hipStream_t st);

hipError_t launch_index_topk(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                             const void* q, const float* w, const void* key_pool, int32_t* sel,
                             float* scores, int64_t ld, void* ws_select, hipStream_t st) {
  hipError_t e;
  if (index_mfma_supported(h->cfg)) {
    RowGroups g;
    RowMap map;
    split_rows(in, &g, &map);
    if (select_lists_used(h, in)) {
      // Every row is scored one per workgroup (decode rows, short spans): that kernel also writes
      // each block's counts and top keys, and one launch selects from them.
      const ScoreHist hs = select_hist_buffers(h, in, ws_select);
      e = launch_index_scores_mfma(h, p, in, map, q, w, key_pool, scores, ld, false, nullptr, 0,
                                   nullptr, 0, &hs, st);
      if (e != hipSuccess) return e;
      return launch_select_lists(h, p, in, scores, ld, sel, ws_select, st);
    }
    int nb_max = 0;
    uint32_t* mm = select_minmax_buffer(h, in, ws_select, &nb_max);
    e = index_scores_mfma_all(h, p, in, q, w, key_pool, scores, ld, false, mm, nb_max, st);
    if (e != hipSuccess) return e;
    return launch_select_topk_ex(h, p, in, scores, ld, sel, ws_select, true, st);
  }
  e = launch_index_scores_generic(h, p, in, q, w, key_pool, scores, ld, false, st);
  if (e != hipSuccess) return e;
  return launch_select_topk_ex(h, p, in, scores, ld, sel, ws_select, false, st);
}

bool attend_mfma_supported(const dsa_config& c);
bool attend_mfma_plan_ok(const DevPlan& p);
size_t attend_mfma_workspace(const dsa_config& c, const PlanInfo& in);
hipError_t launch_attend_mfma(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                              const int32_t* sel, const void* qn, const void* qp, const void* pool,
                              float sm_scale, const float* sink, void* out, void* ws, hipStream_t st);

size_t attend_workspace_bytes(const dsa_handle* h, const PlanInfo& in) {
  return attend_mfma_supported(h->cfg) ? attend_mfma_workspace(h->cfg, in) : 0;
}

hipError_t launch_attend(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                         const int32_t* sel, const void* q_nope, const void* q_pe,
                         const void* latent_pool, float sm_scale, const float* sink, void* out,
                         void* ws, hipStream_t st) {
  if (attend_mfma_supported(h->cfg) && attend_mfma_plan_ok(p))
    return launch_attend_mfma(h, p, in, sel, q_nope, q_pe, latent_pool, sm_scale, sink, out, ws, st);
  return launch_attend_generic(h, p, in, sel, q_nope, q_pe, latent_pool, sm_scale, sink, out, st);
}
