// cbr_plan.cpp -- per-shape kernel plans: the eligibility of each plan, the default rule,
// the compiled-in table of measured plans (the MI355X counterpart of the CBR page's
// empirical engine search, section 7, and of the TileLang page's autotuned tile
// configurations: a winner per shape, found offline by timing every eligible plan), and
// the tuning override.
#include <atomic>

#include "../../include/cbr.h"
#include "cbr_launch.h"

namespace cbr {
namespace {

struct TuneEntry {
    int stage;
    int n, h, w, c, k, r, s, sh, sw, ph, pw;
    int plan;
};

const TuneEntry kTuneTable[] = {
#include "cbr_tune_table.inc"
    {-1, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0},   // end
};

std::atomic<int> g_override[NSTAGES];

bool is_conv_stage(int stage) { return stage == STAGE_TRAIN || stage == STAGE_INFER || stage == STAGE_DGRAD; }

int conv_epilogue(int stage) { return stage == STAGE_TRAIN ? EPI_STATS : stage == STAGE_INFER ? EPI_BIAS_RELU : EPI_PLAIN; }

}  // namespace

bool plan_eligible(const ConvGeom &layer, int stage, int plan)
{
    const ConvGeom g = stage == STAGE_DGRAD ? dgrad_geom(layer) : layer;
    switch (plan) {
    case PLAN_PERSIST3X3: return stage == STAGE_TRAIN && halo_eligible(g);
    case PLAN_FIRST_LAYER: return stage == STAGE_TRAIN && c3s2_eligible(g);
    case PLAN_IG_224X256:
    case PLAN_IG_448X128: return is_conv_stage(stage) && igemm_eligible(g, conv_epilogue(stage), plan);
    case PLAN_GEN_128X128:
    case PLAN_GEN_128X64: return is_conv_stage(stage);
    case PLAN_WG_TR: return stage == STAGE_WGRAD && wgrad_tr_eligible(g);
    case PLAN_WG_GEN: return stage == STAGE_WGRAD;
    case PLAN_WG_TR_WIDE: return stage == STAGE_WGRAD && wgrad_tr_wide_eligible(g);
    case PLAN_BWD_SERIAL: return stage == STAGE_BWD;
    case PLAN_BWD_OVERLAP: return stage == STAGE_BWD && layer.sh == 1 && layer.sw == 1;
    case PLAN_BWD_FUSED: return stage == STAGE_BWD && layer.K <= 256 && layer.C % 8 == 0;
    default: return false;
    }
}

// The rule for shapes without a measured plan: the specialised kernels where they apply;
// the large-tile conv (224 x 256 chunks where K allows, else 448 x 128) when each of its
// at most 256 workgroups gets at least 128 output pixels; else the generic conv (128 x 128
// tiles for K >= 128).  Over the 206 layer/stage timings of the tuning run that wrote
// cbr_tune_table.inc, this rule is within 1% of the per-shape best in total time; the
// persistent large-tile conv loses badly when few pixels per workgroup meet many channel
// chunks (up to 18x on a 7x7 layer with 2048 output channels).
int default_plan(const ConvGeom &layer, int stage)
{
    if (stage == STAGE_WGRAD) return wgrad_tr_eligible(layer) ? PLAN_WG_TR : PLAN_WG_GEN;
    if (stage == STAGE_BWD) return PLAN_BWD_SERIAL;
    if (stage == STAGE_TRAIN && halo_eligible(layer)) return PLAN_PERSIST3X3;
    if (stage == STAGE_TRAIN && c3s2_eligible(layer)) return PLAN_FIRST_LAYER;
    const ConvGeom g = stage == STAGE_DGRAD ? dgrad_geom(layer) : layer;
    const int grid = std::min(256, (g.M + 31) / 32);
    const int rows_per_wg = (g.M + grid - 1) / grid;
    if (rows_per_wg >= 128) {
        if (plan_eligible(layer, stage, PLAN_IG_224X256)) return PLAN_IG_224X256;
        if (plan_eligible(layer, stage, PLAN_IG_448X128)) return PLAN_IG_448X128;
    }
    return g.K >= 128 ? PLAN_GEN_128X128 : PLAN_GEN_128X64;
}

int resolve_plan(const ConvGeom &g, int stage)
{
    const int ov = g_override[stage].load(std::memory_order_relaxed);
    if (ov != PLAN_DEFAULT && plan_eligible(g, stage, ov)) return ov;
    for (const TuneEntry *e = kTuneTable; e->stage >= 0; ++e)
        if (e->stage == stage && e->n == g.N && e->h == g.H && e->w == g.W && e->c == g.C && e->k == g.K &&
            e->r == g.R && e->s == g.S && e->sh == g.sh && e->sw == g.sw && e->ph == g.ph && e->pw == g.pw &&
            plan_eligible(g, stage, e->plan))
            return e->plan;
    return default_plan(g, stage);
}

const char *plan_name(int plan)
{
    switch (plan) {
    case PLAN_DEFAULT: return "default";
    case PLAN_PERSIST3X3: return "persistent_3x3_c64";
    case PLAN_FIRST_LAYER: return "first_layer_c3s2";
    case PLAN_IG_224X256: return "large_tile_224x256";
    case PLAN_IG_448X128: return "large_tile_448x128";
    case PLAN_GEN_128X128: return "generic_128x128";
    case PLAN_GEN_128X64: return "generic_128x64";
    case PLAN_WG_TR: return "wgrad_transposed_read";
    case PLAN_WG_GEN: return "wgrad_generic";
    case PLAN_WG_TR_WIDE: return "wgrad_transposed_read_256x256";
    case PLAN_BWD_SERIAL: return "backward_serial";
    case PLAN_BWD_OVERLAP: return "backward_wgrad_beside_dgrad";
    case PLAN_BWD_FUSED: return "backward_dz_formed_in_gradients";
    default: return "unknown";
    }
}

bool set_plan_override(int stage, int plan)
{
    if (stage < 0 || stage >= NSTAGES || plan < 0 || plan >= NPLANS) return false;
    g_override[stage].store(plan, std::memory_order_relaxed);
    return true;
}

}  // namespace cbr
