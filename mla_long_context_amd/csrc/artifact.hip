// Validation of an offline Local-head artifact before reuse (RedKnot-MLA,
// section 2, "Canonical offline artifacts": a document is processed alone at
// canonical position zero, its Local-head results are kept, and reuse falls
// back to full recomputation when a layer is missing, the tokens or the
// profile differ, or the generation is stale). Host code only: the decision
// is taken before any kernel of the reuse path is launched.
#include "mla_internal.h"

extern "C" uint64_t mla_token_hash(const int32_t* tokens, int64_t n) {
  // 64-bit FNV-1a over the ids' little-endian bytes
  uint64_t h = 0xcbf29ce484222325ull;
  if (!tokens) return h;
  for (int64_t i = 0; i < n; ++i) {
    const uint32_t t = static_cast<uint32_t>(tokens[i]);
    for (int b = 0; b < 4; ++b) {
      h ^= (t >> (8 * b)) & 0xffu;
      h *= 0x100000001b3ull;
    }
  }
  return h;
}

namespace {

bool same_profile(const mla_artifact_meta& a, const mla_artifact_meta& r) {
  return a.n_heads == r.n_heads && a.n_local == r.n_local && a.d_c == r.d_c && a.d_rope == r.d_rope &&
         a.d_nope == r.d_nope && a.d_v == r.d_v && a.rope_base == r.rope_base && a.n_layers == r.n_layers;
}

}  // namespace

extern "C" int mla_artifact_check(const mla_artifact_meta* artifact, const mla_artifact_meta* request,
                                  int* reason) {
  mla_clear_error();
  MLA_REQUIRE(artifact && request && reason, MLA_ERR_INVALID_ARG, "mla_artifact_check: null pointer argument");
  MLA_REQUIRE(artifact->n_layers >= 0 && artifact->n_layers <= 64 && request->n_layers >= 0 &&
                  request->n_layers <= 64,
              MLA_ERR_INVALID_ARG, "mla_artifact_check: layer counts must be in 0..64 (got %d, %d)",
              artifact->n_layers, request->n_layers);
  const mla_artifact_meta& a = *artifact;
  const mla_artifact_meta& r = *request;
  // every layer the request needs must be present
  if ((r.layer_mask & ~a.layer_mask) != 0) {
    *reason = MLA_ARTIFACT_MISSING_LAYER;
  } else if (a.n_tokens != r.n_tokens || a.token_hash != r.token_hash) {
    *reason = MLA_ARTIFACT_TOKEN_MISMATCH;
  } else if (!same_profile(a, r)) {
    *reason = MLA_ARTIFACT_PROFILE_MISMATCH;
  } else if (a.generation != r.generation) {
    *reason = MLA_ARTIFACT_STALE;
  } else {
    *reason = MLA_ARTIFACT_VALID;
  }
  return MLA_OK;
}
