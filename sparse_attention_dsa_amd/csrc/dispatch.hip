// Kernel choice per configuration and plan.
#include "dsa_internal.hpp"

hipError_t launch_index_scores_generic(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                                       const void* q, const float* w, const void* pool,
                                       float* scores, int64_t ld, bool fill, hipStream_t st);
hipError_t launch_attend_generic(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                                 const int32_t* sel, const void* qn, const void* qp,
                                 const void* pool, float sm_scale, void* out, hipStream_t st);

hipError_t launch_index_scores(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                               const void* q, const float* w, const void* key_pool, float* scores,
                               int64_t ld, bool fill_masked, hipStream_t st) {
  return launch_index_scores_generic(h, p, in, q, w, key_pool, scores, ld, fill_masked, st);
}

size_t attend_workspace_bytes(const dsa_handle*, const PlanInfo&) { return 0; }

hipError_t launch_attend(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                         const int32_t* sel, const void* q_nope, const void* q_pe,
                         const void* latent_pool, float sm_scale, void* out, void*, hipStream_t st) {
  return launch_attend_generic(h, p, in, sel, q_nope, q_pe, latent_pool, sm_scale, out, st);
}
