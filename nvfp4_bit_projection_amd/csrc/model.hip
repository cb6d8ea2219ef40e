// model.hip -- one whole decode step: per layer the attention (attn.hip), then
// the dense MLP (attn.hip) or the MoE layer (kernels.hip), each reading the
// residual stream through a unit-gain RMSNorm folded into its first kernel
// and adding its output back into the residual in its last one; then the
// NVFP4 head with argmax.
//
// Layer plan [P2 "Recursive Releases Flint, a 40B MoE Coding Model That Runs
// Locally at 125 Tokens per Second", "How does Flint's architecture work?":
// 49 layers, 2 dense then 47 MoE; 35 sliding-window and 14 full-attention
// layers].
#include "../../include/flint_model.h"
#include "flint_common.h"
#include "flint_internal.h"

namespace flint {
namespace {

__global__ __launch_bounds__(256) void k_copy_vec(const float* __restrict__ s, float* __restrict__ d, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) d[i] = s[i];
}

// persist: the persistent MoE kernel's exchange area (control words first),
// kept from call to call; scratch: shared by the layers in turn
struct ModelWs {
  size_t persist, h, scratch, total;
  ModelWs(size_t scratch_bytes, bool persistent) {
    size_t o = 0;
    persist = o; o = align_up(o + (persistent ? stack_persistent_ws_bytes() : 0), 256);
    h = o; o = align_up(o + 4 * (size_t)kHidden, 256);
    scratch = o; o = align_up(o + scratch_bytes, 256);
    total = o;
  }
};

// the scratch the layers and the head need in turn (they run one after the
// other on one stream, so they share it); 0 if the model is invalid
size_t model_scratch(const flint_model* m) {
  if (!m || m->n_layers < 1 || m->n_dense < 0 || m->n_dense > m->n_layers || !m->is_full || !m->attn ||
      !m->k_cache || !m->v_cache || !m->cap || (m->n_dense > 0 && !m->dense) ||
      (m->n_dense < m->n_layers && !m->moe_layers) || m->vocab < 1)
    return 0;
  size_t s = HeadWs(1).total;
  const size_t a0 = flint_attn_workspace_bytes(&m->sliding), a1 = flint_attn_workspace_bytes(&m->full);
  if (a0 == 0 || a1 == 0) return 0;
  s = s > a0 ? s : a0;
  s = s > a1 ? s : a1;
  if (m->n_dense > 0) s = s > 4 * (size_t)m->dense_width ? s : 4 * (size_t)m->dense_width;
  if (m->n_dense < m->n_layers) {
    if (api_moe_check(&m->moe, &m->moe_layers[0]) != FLINT_OK) return 0;
    const size_t mw = api_moe_ws_bytes(m->moe);
    s = s > mw ? s : mw;
  }
  return s;
}

// the optional plan of the MoE layers matches the model and allows the
// persistent schedule
int32_t check_moe_plan(const flint_model* m) {
  const flint_stack_plan* p = m->moe_plan;
  if (!p) return FLINT_OK;
  if (!p->table || !p->packed) return FLINT_E_NULL;
  const flint_moe_dims &a = p->dims, &b = m->moe;
  if (a.hidden != b.hidden || a.n_experts != b.n_experts || a.expert_width != b.expert_width ||
      a.top_k != b.top_k || a.shared_width != b.shared_width || p->n_layers != m->n_layers - m->n_dense)
    return FLINT_E_DIMS;
  return stack_persistent_supported(a, 1) ? FLINT_OK : FLINT_E_UNSUPPORTED;
}

}  // namespace
}  // namespace flint

using namespace flint;

extern "C" {

size_t flint_model_workspace_bytes(const flint_model* m) {
  const size_t s = model_scratch(m);
  return s ? ModelWs(s, m->moe_plan != nullptr).total : 0;
}

int32_t flint_model_decode(const flint_model* m, const float* x, int32_t pos, float* logits_opt, int32_t* argmax,
                           float* h_out_opt, void* ws, size_t ws_bytes, void* stream) {
  if (!m || !x || !argmax || !ws) return FLINT_E_NULL;
  const size_t scratch = model_scratch(m);
  if (scratch == 0) return FLINT_E_DIMS;
  if (m->moe.hidden != kHidden || m->sliding.hidden != kHidden || m->full.hidden != kHidden)
    return FLINT_E_UNSUPPORTED;
  if (!(m->eps >= 0.0f) || pos < 0) return FLINT_E_DIMS;
  int32_t st;
  for (int l = 0; l < m->n_layers; ++l) {
    if (m->is_full[l] != 0 && m->is_full[l] != 1) return FLINT_E_DIMS;
    const flint_attn_dims* ad = m->is_full[l] ? &m->full : &m->sliding;
    if ((st = attn_check(ad, &m->attn[l], pos, m->k_cache[l], m->v_cache[l], m->cap[l]))) return st;
    if (l < m->n_dense) {
      const flint_nvfp4* dn = m->dense + 3 * l;
      if ((st = dense_check(dn, dn + 1, dn + 2, kHidden, m->dense_width))) return st;
    } else if ((st = api_moe_check(&m->moe, &m->moe_layers[l - m->n_dense]))) {
      return st;
    }
  }
  if ((st = check_moe_plan(m))) return st;
  if (!m->head.codes || !m->head.scales || !m->head.tscale) return FLINT_E_NULL;
  if (((uintptr_t)x & 15) || ((uintptr_t)ws & 15) || ((uintptr_t)m->head.codes & 15) ||
      ((uintptr_t)argmax & 3) || ((uintptr_t)logits_opt & 3) || ((uintptr_t)h_out_opt & 3))
    return FLINT_E_ALIGN;
  const ModelWs w(scratch, m->moe_plan != nullptr);
  if (ws_bytes < w.total) return FLINT_E_WORKSPACE;
  if ((st = api_check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  char* base = static_cast<char*>(ws);
  float* h = reinterpret_cast<float*>(base + w.h);
  void* sc = base + w.scratch;
  k_copy_vec<<<8, 256, 0, s>>>(x, h, kHidden);
  hipError_t e = hipGetLastError();
  bool qkv_ready = false;  // this layer's q, k, v were computed by the kernel before
  for (int l = 0; l < m->n_layers && e == hipSuccess; ++l) {
    const flint_attn_dims& ad = m->is_full[l] ? m->full : m->sliding;
    e = attn_run(ad, m->attn[l], h, m->eps, pos, m->k_cache[l], m->v_cache[l], m->cap[l], h, true, sc, s,
                 qkv_ready);
    qkv_ready = false;
    if (e != hipSuccess) break;
    if (l < m->n_dense) {
      const flint_nvfp4* dn = m->dense + 3 * l;
      e = dense_run(dn[0], dn[1], dn[2], m->dense_width, h, m->eps, h, true, sc, s);
    } else if (m->moe_plan) {
      // one launch of the persistent kernel: layer l - n_dense of the plan's
      // table, no head, the residual updated in place.  Every workgroup
      // copies h into LDS before its first exchange store, and the
      // workgroups that write h_out do so only after the layer's residual
      // exchange, which needs the partial outputs of all 256 workgroups (each
      // owns 64 of the 2,048 rows in every XCD); so no store to h can
      // overtake a read of it, whatever the number of experts.  The launch
      // also applies the next layer's q, k, v projections to the norm of the
      // new residual, which it holds in every workgroup
      StackQkv nx{};
      const bool next = l + 1 < m->n_layers;
      if (next) {
        const flint_attn_dims& an = m->is_full[l + 1] ? m->full : m->sliding;
        const flint_attn_layer& A = m->attn[l + 1];
        const flint_nvfp4* mats[3] = {&A.q, &A.k, &A.v};
        for (int i = 0; i < 3; ++i) {
          nx.codes[i] = mats[i]->codes;
          nx.scales[i] = mats[i]->scales;
          nx.tscale[i] = mats[i]->tscale;
        }
        nx.rows[0] = an.n_q_heads * an.head_dim;
        nx.rows[1] = nx.rows[2] = an.n_kv_heads * an.head_dim;
        nx.out = reinterpret_cast<float*>(static_cast<char*>(sc) + attn_qkv_offset(an));
      }
      e = launch_stack_persistent(m->moe, 1, 0, m->moe_plan->table, h, 1, m->eps, nullptr, nullptr, nullptr,
                                  base + w.persist, nullptr, s, l - m->n_dense, h, next ? &nx : nullptr);
      qkv_ready = next;
    } else {
      e = api_moe_run(m->moe, m->moe_layers[l - m->n_dense], h, m->eps, h, true, sc, s);
    }
  }
  if (e == hipSuccess) {
    const HeadWs hw(1);
    e = launch_lmhead(m->head, m->vocab, h, 1, m->eps, logits_opt, argmax,
                      reinterpret_cast<HeadPartial*>(static_cast<char*>(sc) + hw.partials), s);
  }
  if (e == hipSuccess && h_out_opt) {
    k_copy_vec<<<8, 256, 0, s>>>(h, h_out_opt, kHidden);
    e = hipGetLastError();
  }
  return e == hipSuccess ? FLINT_OK : api_hip_fail(e);
}

int32_t flint_model_error(const flint_model* m, const void* ws, size_t ws_bytes, int32_t* error) {
  if (!m || !ws || !error) return FLINT_E_NULL;
  const size_t scratch = model_scratch(m);
  if (scratch == 0) return FLINT_E_DIMS;
  const ModelWs w(scratch, m->moe_plan != nullptr);
  if (ws_bytes < w.total) return FLINT_E_WORKSPACE;
  *error = 0;
  if (!m->moe_plan) return FLINT_OK;
  int32_t st = api_check_device();
  if (st) return st;
  const hipError_t e = read_stack_error(static_cast<const char*>(ws) + w.persist, error);
  return e == hipSuccess ? FLINT_OK : api_hip_fail(e);
}

}  // extern "C"
