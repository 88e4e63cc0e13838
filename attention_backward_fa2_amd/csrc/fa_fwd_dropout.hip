// fa_fwd_dropout.hip -- the dropout instantiations of the forward kernel of
// fa_fwd.hip, in a translation unit of their own so that they compile in
// parallel with the rest.
#define FA_TU_DROPOUT 1
#include "fa_fwd.hip"
