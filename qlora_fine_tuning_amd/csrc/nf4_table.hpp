// fp32 bit patterns of the 16 NF4 levels, ascending (level 0 = -1, level 7 =
// exact 0, level 15 = +1). Construction: asymmetric normal-quantile table;
// the 8 positive levels are Phi^-1(1/2 + (delta - 1/2) j / 8), j = 1..8, the
// 7 negative levels -Phi^-1(1/2 + (delta - 1/2) j / 7), j = 1..7, all divided
// by Phi^-1(delta) and rounded once to fp32. delta = ((1 - 1/30) + (1 - 1/32))
// / 2, the mean of the outermost bin centres of 15 and 16 equal-probability
// bins (the offset of the QLoRA paper's NF4 construction).
#pragma once
#define QLORA_NF4_LEVEL_BITS                                                  \
  0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu, 0xbe91a24bu,            \
      0xbe3d353du, 0xbdba7869u, 0x00000000u, 0x3da2fb01u, 0x3e24cadfu,        \
      0x3e7c04dau, 0x3ead0336u, 0x3ee1a4b5u, 0x3f1007a9u, 0x3f3913b0u,        \
      0x3f800000u
