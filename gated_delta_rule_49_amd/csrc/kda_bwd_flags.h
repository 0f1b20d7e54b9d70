// kda_bwd_flags.h -- launch flags of the backward, beside the prologue bits of kda_common.h
// (KDA_PRO_GATE 1, KDA_PRO_NORM 2, KDA_STATES_ONLY 4), in the same flag words.
#pragma once

namespace kda {

// The caller passes the states at every 32-token boundary, so they are neither recomputed nor held
// in the workspace.
constexpr int KDA_BWD_STATES_GIVEN = 8;
// The batch suits the state-gradient scan with one workgroup per chain (sequences of nearly equal
// length, enough chains to fill the chip), used where the error budget is bf16's at d = 128.
constexpr int KDA_BWD_ONE_WG_SCAN = 32;

}  // namespace kda
