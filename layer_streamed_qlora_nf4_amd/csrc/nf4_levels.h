// The 16 NormalFloat-4 levels, float32, ascending.
//
// NF4 is named by the pages as the streamed base's quantisation (About;
// LS-docs "Turn it on") without its levels.  These are the levels of the
// QLoRA NormalFloat-4 construction: normal quantiles at equally spaced
// probabilities, 8 above zero and 7 below it, an exact zero, scaled so the
// extremes are -1 and +1, each rounded once to float32.
#pragma once

namespace lsq {
constexpr float kNF4Levels[16] = {
    -1.0f,           -0x1.647362p-1f, -0x1.0cd65cp-1f, -0x1.94653cp-2f,
    -0x1.234496p-2f, -0x1.7a6a7ap-3f, -0x1.74f0d2p-4f, 0.0f,
    0x1.45f602p-4f,  0x1.4995bep-3f,  0x1.f809b4p-3f,  0x1.5a066cp-2f,
    0x1.c3496ap-2f,  0x1.200f52p-1f,  0x1.722760p-1f,  1.0f};
static __constant__ const float kNF4LevelsDev[16] = {
    -1.0f,           -0x1.647362p-1f, -0x1.0cd65cp-1f, -0x1.94653cp-2f,
    -0x1.234496p-2f, -0x1.7a6a7ap-3f, -0x1.74f0d2p-4f, 0.0f,
    0x1.45f602p-4f,  0x1.4995bep-3f,  0x1.f809b4p-3f,  0x1.5a066cp-2f,
    0x1.c3496ap-2f,  0x1.200f52p-1f,  0x1.722760p-1f,  1.0f};
}  // namespace lsq
