// validate.cpp -- the argument checks of the C ABI that need no device: hyper-
// parameters, the loss-scaling rule, the precision descriptor and the list
// header.  The per-tensor pointer, alignment and shard checks are made by the
// planner (build_plan), which walks the list anyway.
#include <cmath>

#include "plan.hpp"

namespace adamw {

adamw_status check_hparams(const adamw_hparams* hp, std::string& err)
{
    if (!hp) { err = "hparams is null"; return ADAMW_E_INVALID; }
    const float v[6] = {hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->inv_loss_scale};
    for (float x : v)
        if (!std::isfinite(x)) { err = "hyper-parameters must be finite"; return ADAMW_E_INVALID; }
    if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f)) {
        err = "beta1 and beta2 must lie in [0, 1)";
        return ADAMW_E_INVALID;
    }
    if (hp->eps < 0.0f) { err = "eps < 0"; return ADAMW_E_INVALID; }
    if (hp->lr < 0.0f) { err = "lr < 0"; return ADAMW_E_INVALID; }
    if (hp->weight_decay < 0.0f) { err = "weight_decay < 0"; return ADAMW_E_INVALID; }
    if (!(hp->inv_loss_scale > 0.0f)) { err = "inv_loss_scale must be > 0"; return ADAMW_E_INVALID; }
    return ADAMW_OK;
}

adamw_status check_scaler(const adamw_loss_scaler* sc, std::string& err)
{
    if (!sc) { err = "loss scaler is null"; return ADAMW_E_INVALID; }
    if (!std::isfinite(sc->growth_factor) || !(sc->growth_factor >= 1.0f)) {
        err = "growth_factor must be finite and >= 1";
        return ADAMW_E_INVALID;
    }
    if (!(sc->backoff_factor > 0.0f && sc->backoff_factor <= 1.0f)) {
        err = "backoff_factor must lie in (0, 1]";
        return ADAMW_E_INVALID;
    }
    if (sc->growth_interval < 1) { err = "growth_interval must be >= 1"; return ADAMW_E_INVALID; }
    return ADAMW_OK;
}

adamw_status basic_list_check(const adamw_tensor_list* list, std::string& err)
{
    if (!list) { err = "tensor list is null"; return ADAMW_E_INVALID; }
    if (list->n_tensors < 0) { err = "n_tensors < 0"; return ADAMW_E_INVALID; }
    if (list->n_tensors > 0 && !list->numel) { err = "numel array is null"; return ADAMW_E_INVALID; }
    return ADAMW_OK;
}

adamw_status check_pure_precision(const adamw_pure_precision* prec, std::string& err)
{
    if (!prec) { err = "precision descriptor is null"; return ADAMW_E_INVALID; }
    const bool ok_m = prec->exp_avg == ADAMW_F32 || prec->exp_avg == ADAMW_BF16;
    const bool ok_v = prec->exp_avg_sq == ADAMW_F32 || prec->exp_avg_sq == ADAMW_BF16;
    if (!ok_m || !ok_v) {
        err = "exp_avg / exp_avg_sq dtype must be ADAMW_F32 or ADAMW_BF16";
        return ADAMW_E_UNSUPPORTED;
    }
    if (prec->kahan != ADAMW_KAHAN_NONE && prec->kahan != ADAMW_KAHAN_BF16 && prec->kahan != ADAMW_KAHAN_F32) {
        err = "kahan must be ADAMW_KAHAN_NONE, ADAMW_KAHAN_BF16 or ADAMW_KAHAN_F32";
        return ADAMW_E_INVALID;
    }
    return ADAMW_OK;
}

}  // namespace adamw
